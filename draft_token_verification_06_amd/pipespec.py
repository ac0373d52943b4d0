"""Asynchronous k-stage speculative pipeline driven through the verification
library: a discrete-time simulation of PipeSpec's producer/consumer stages.

Source: "PipeSpec: Breaking Stage Dependencies in Hierarchical LLM Decoding"
(Pith review page).  From "What carries the argument": k models of increasing
size, each writing to its own buffer O_i; M_0 drafts continuously; M_i (i >= 1)
takes the drafts in O_{i-1}, makes its own single-token predictions, appends
the longest matching prefix (plus its own next token) to O_i, and on a
mismatch rolls the earlier buffers back to the last verified token.  From
"Core claim": the steady-state verification probability
rho = alpha / (1 - alpha^(gamma+1) + alpha) and E[N] of Eq. (4).  From "What
would settle it": the final verifier's buffer occupancy when it starts a step,
and the token rate at alpha near 0.05.

Every stage step is one batched call of the library over all streams:
sv_verify_greedy (temperature 0, the page's setting) or sv_verify_window
(speculative sampling), with the window length of each stream set to the
drafts it has pending; a window length of 0 makes the stage emit its own next
token (argmax of, or a draw from, its row 0).  Buffer hand-offs are
sv_rollback calls.  The synthetic models are deterministic functions of the
context (HashModels), so the greedy pipeline's output can be checked against
the last model's own greedy sequence.

Time model (the page gives none; readings):
* stage i's step takes costs[i] time units, verification or single token alike
  (decoding is memory-bound), plus verify_cost * window_len if set;
* every stage starts its next step as soon as its previous one ends;
* a step reads its inputs when it starts and applies its output when it ends;
  an output whose own buffer was rolled back in between is discarded;
* steps ending at the same instant are applied from the last stage to the first,
  then all of them start again;
* stage 0 drafts one token per step and stops while it is `lookahead` tokens
  ahead of stage 1;
* uniforms of speculative sampling are keyed per stage and step (tag), per
  stream (seq_id) and per position (base_pos), so no decision reuses another's.
"""
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_GOLD = np.uint64(0x9E3779B97F4A7C15)


def _mix_np(x):
    """SplitMix64 finaliser on numpy uint64 (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = x ^ (x >> np.uint64(30))
        x = x * _M1
        x = x ^ (x >> np.uint64(27))
        x = x * _M2
        x = x ^ (x >> np.uint64(31))
    return x


def _as_i64(c):
    c = int(c) & 0xFFFFFFFFFFFFFFFF
    return c - (1 << 64) if c >= (1 << 63) else c


def _lsr(x, s):
    return (x >> s) & ((1 << (64 - s)) - 1)


def _mix_t(x):
    """The same finaliser on int64 torch tensors (two's-complement wrap)."""
    x = x ^ _lsr(x, 30)
    x = x * _as_i64(_M1)
    x = x ^ _lsr(x, 27)
    x = x * _as_i64(_M2)
    x = x ^ _lsr(x, 31)
    return x


def context_key(prev_key, token):
    """Key of a context extended by one token."""
    with np.errstate(over="ignore"):
        return _mix_np(np.asarray(prev_key, dtype=np.uint64) ^ ((np.asarray(token, dtype=np.uint64)
                                                                 + np.uint64(1)) * _GOLD))


def root_key(stream_seed):
    return _mix_np(np.uint64(stream_seed) + _GOLD)


class HashModels:
    """Synthetic language models M_0..M_{K-1} over V tokens.

    Logits of M_i at a context with key k: scale * N_0(k) + sigmas[i] * N_{i+1}(k),
    where N_j(k) is a vector of V independent standard normals drawn from a
    counter-based hash of (k, j, token) (Box-Muller on two 24-bit uniforms).
    Each model is a deterministic function of the context; models with small
    sigmas agree more often."""

    def __init__(self, V, sigmas: Sequence[float], scale=3.0, device="cpu", dtype=torch.bfloat16):
        self.V = V
        self.sigmas = list(sigmas)
        self.scale = scale
        self.device = device
        self.dtype = dtype
        self._tok = torch.arange(V, device=device, dtype=torch.int64)

    def _normals(self, keys, j):
        k = keys.view(-1, 1)
        base = k + _as_i64((j + 1) * int(_GOLD)) + self._tok.view(1, -1) * _as_i64(_M2)
        h1 = _mix_t(base)
        h2 = _mix_t(h1 ^ _as_i64(_GOLD))
        u1 = (_lsr(h1, 40).to(torch.float32) + 0.5) * 2.0 ** -24
        u2 = _lsr(h2, 40).to(torch.float32) * 2.0 ** -24
        return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * np.pi * u2)

    def logits(self, i, keys):
        """(len(keys), V) logits of model i; keys: uint64 numpy array."""
        kt = torch.from_numpy(np.asarray(keys, dtype=np.uint64).view(np.int64).copy()).to(self.device)
        x = self.scale * self._normals(kt, 0)
        if self.sigmas[i] != 0.0:
            x = x + self.sigmas[i] * self._normals(kt, i + 1)
        return x.to(self.dtype)


class LibraryVerifier:
    """Stage steps through the HIP library (sv_verify_greedy / sv_verify_window)
    and buffer hand-offs through sv_rollback."""

    def __init__(self):
        from . import api
        self.api = api

    def step(self, mode, target, draft, tokens, window_len, *, seed, tag, seq_ids, base_pos):
        if mode == "greedy":
            r = self.api.verify_greedy(target, tokens, window_len=window_len)
        else:
            r = self.api.verify_window(target, draft, tokens, seed=seed, tag=tag, window_len=window_len,
                                       seq_ids=seq_ids, base_pos=base_pos)
        return r.n_accepted, r.out_tokens

    def rollback(self, buf, lens, stage, verified, verified_len):
        self.api.rollback(buf, lens, stage, verified, verified_len)


@dataclass
class PipeConfig:
    costs: Sequence[int]           # time units per step of M_0..M_{K-1}
    gammas: Sequence[int]          # window of M_1..M_{K-1}
    sigmas: Sequence[float]        # model noise (HashModels)
    V: int = 32000
    streams: int = 64
    mode: str = "greedy"
    lookahead: Optional[int] = None  # stage-0 drafts past stage 1 (default 4 * gammas[0])
    cap: int = 2048
    seed: int = 0
    verify_cost: float = 0.0       # extra time per window token of a verification step
    dtype: torch.dtype = torch.bfloat16
    shared_prompt: bool = False    # every stream starts from the same context


@dataclass
class StageStats:
    steps: int = 0
    discarded: int = 0
    verify_steps: int = 0
    emitted: int = 0
    accepted: int = 0
    tested: int = 0
    full_windows: int = 0
    next_tests: int = 0     # own token met a waiting draft (after a single token or a bonus)
    next_matches: int = 0
    occupancy: list = field(default_factory=list)  # histogram of window_len at step start


class PipeSpecSim:
    """Discrete-time simulation of a k-stage PipeSpec pipeline over S streams."""

    def __init__(self, cfg: PipeConfig, device="cuda", verifier=None, models=None):
        K = len(cfg.costs)
        if K < 2 or len(cfg.gammas) != K - 1 or len(cfg.sigmas) != K:
            raise ValueError("costs and sigmas need one entry per model, gammas one per verifier")
        if any(int(c) < 1 for c in cfg.costs) or any(g < 1 for g in cfg.gammas):
            raise ValueError("costs and gammas must be positive")
        self.cfg = cfg
        self.K = K
        self.S = cfg.streams
        self.dev = device
        self.ver = verifier if verifier is not None else LibraryVerifier()
        self.models = models if models is not None else HashModels(cfg.V, cfg.sigmas, device=device,
                                                                   dtype=cfg.dtype)
        self.lookahead = cfg.lookahead if cfg.lookahead is not None else 4 * cfg.gammas[0]
        S, cap = self.S, cfg.cap
        self.buf = torch.zeros(S, K, cap, dtype=torch.int32, device=device)
        self.lens = torch.zeros(S, K, dtype=torch.int32, device=device)
        self.h_buf = np.zeros((S, K, cap), dtype=np.int32)
        self.h_len = np.zeros((S, K), dtype=np.int64)
        self.version = np.zeros((S, K), dtype=np.int64)
        ids = np.zeros(S, dtype=np.uint64) if cfg.shared_prompt else np.arange(S, dtype=np.uint64)
        self.roots = root_key(ids + np.uint64(cfg.seed) * np.uint64(1 << 20))
        self._kcache = {}  # (stream, stage) -> (prefix keys, tokens they were computed from)
        self.stats = [StageStats(occupancy=[0] * (g + 1)) for g in [0] + list(cfg.gammas)]
        self.time = 0
        self.steps_started = [0] * K
        self.inflight = [None] * K
        self.ends = [0] * K

    # -- host mirror and context keys -------------------------------------
    def _sync(self):
        self.h_buf = self.buf.cpu().numpy()
        self.h_len = self.lens.cpu().numpy().astype(np.int64)

    def _prefix_keys(self, s, i, upto):
        """Keys of buffer i's prefixes of length 0..upto; the cached keys are
        kept up to the first token that changed since they were computed."""
        ks, kt = self._kcache.get((s, i), ([self.roots[s]], np.zeros(0, dtype=np.int32)))
        toks = self.h_buf[s, i]
        n = min(len(kt), upto)
        diff = np.nonzero(kt[:n] != toks[:n])[0]
        good = int(diff[0]) if diff.size else n
        del ks[good + 1:]
        for p in range(good, upto):
            ks.append(context_key(ks[p], toks[p]))
        self._kcache[(s, i)] = (ks, toks[:upto].copy())
        return ks

    def _window_keys(self, s, i, L, window):
        """Keys of buffer i's first L tokens extended by window[:j], j = 0..len(window)."""
        k = self._prefix_keys(s, i, L)[L]
        out = [k]
        for t in window:
            k = context_key(k, t)
            out.append(k)
        return out

    # -- steps ---------------------------------------------------------------
    def _start(self, i):
        cfg = self.cfg
        S = self.S
        self.steps_started[i] += 1
        tag = (i << 32) | self.steps_started[i]
        sid = torch.arange(S, dtype=torch.int64, device=self.dev)
        if i == 0:
            ahead = self.h_len[:, 0] - self.h_len[:, 1]
            active = (ahead < self.lookahead) & (self.h_len[:, 0] + 1 <= cfg.cap)
            keys = np.array([self._prefix_keys(s, 0, int(self.h_len[s, 0]))[int(self.h_len[s, 0])]
                             for s in range(S)], dtype=np.uint64)
            row = self.models.logits(0, keys).view(S, 1, -1)
            target = torch.cat([row, torch.zeros_like(row)], dim=1).contiguous()
            draft = torch.zeros_like(row) if cfg.mode != "greedy" else None
            toks = torch.zeros(S, 1, dtype=torch.int32, device=self.dev)
            wl = torch.zeros(S, dtype=torch.int32, device=self.dev)
            base = torch.from_numpy(self.h_len[:, 0].copy()).to(self.dev)
            n, out = self.ver.step(cfg.mode, target, draft, toks, wl, seed=cfg.seed, tag=tag,
                                   seq_ids=sid, base_pos=base)
            self.inflight[0] = {"version": self.version[:, 0].copy(), "active": active,
                                "y": out[:, 0].cpu().numpy()}
        else:
            g = cfg.gammas[i - 1]
            L = self.h_len[:, i]
            active = L + 1 <= cfg.cap
            pending = np.maximum(self.h_len[:, i - 1] - L, 0)
            wl = np.minimum(np.minimum(pending, g), np.maximum(cfg.cap - 1 - L, 0))
            window = np.zeros((S, g), dtype=np.int32)
            tkeys, dkeys = [], []
            for s in range(S):
                w = self.h_buf[s, i - 1, L[s]:L[s] + wl[s]]
                window[s, :wl[s]] = w
                ks = self._window_keys(s, i, int(L[s]), window[s])
                tkeys.extend(ks)
                dkeys.extend(ks[:g])
            target = self.models.logits(i, np.array(tkeys, dtype=np.uint64)).view(S, g + 1, -1)
            draft = None
            if cfg.mode != "greedy":
                draft = self.models.logits(i - 1, np.array(dkeys, dtype=np.uint64)).view(S, g, -1)
            toks = torch.from_numpy(window).to(self.dev)
            wlt = torch.from_numpy(wl.astype(np.int32)).to(self.dev)
            base = torch.from_numpy((L - 1).astype(np.int64)).to(self.dev)
            n, out = self.ver.step(cfg.mode, target, draft, toks, wlt, seed=cfg.seed, tag=tag,
                                   seq_ids=sid, base_pos=base)
            self.inflight[i] = {"version": self.version[:, i].copy(), "active": active, "wl": wl, "window": window,
                                "n": n.cpu().numpy(), "out": out.cpu().numpy()}
        dur = cfg.costs[i]
        if i > 0 and cfg.verify_cost:
            dur = cfg.costs[i] + int(round(cfg.verify_cost * float(np.max(self.inflight[i]["wl"]))))
        self.ends[i] = self.time + dur

    def _apply(self, i):
        st = self.stats[i]
        f = self.inflight[i]
        S = self.S
        live = f["version"] == self.version[:, i]
        if i == 0:
            live &= f["active"]
            idx = np.nonzero(live)[0]
            if idx.size:
                pos = self.h_len[idx, 0]
                sel = torch.from_numpy(idx).to(self.dev)
                self.buf[sel, 0, torch.from_numpy(pos).to(self.dev)] = torch.from_numpy(
                    f["y"][idx].astype(np.int32)).to(self.dev)
                self.lens[sel, 0] += 1
            st.steps += S
            st.discarded += int(S - idx.size)
            self._sync()
            return
        wl, n, out, window = f["wl"], f["n"], f["out"], f["window"]
        live &= f["active"]
        st.steps += S
        st.discarded += int(np.sum(~live))
        for s in np.nonzero(live)[0]:
            L = int(self.h_len[s, i])
            k = int(n[s])
            if k == int(wl[s]) and int(self.h_len[s, i - 1]) > L + k:
                # the stage's own token (single token or bonus) against the draft waiting there
                st.next_tests += 1
                st.next_matches += int(self.h_buf[s, i - 1, L + k] == out[s, k])
            new = list(window[s, :k]) + [int(out[s, k])]
            self.h_buf[s, i, L:L + k + 1] = new
            self.h_len[s, i] = L + k + 1
            st.occupancy[int(wl[s])] += 1
            st.verify_steps += int(wl[s] > 0)
            st.full_windows += int(wl[s] == len(st.occupancy) - 1)
            st.emitted += k + 1
            st.accepted += k
            st.tested += min(k + 1, int(wl[s]))
        self.buf[:, i, :] = torch.from_numpy(self.h_buf[:, i, :]).to(self.dev)
        self.lens[:, i] = torch.from_numpy(self.h_len[:, i].astype(np.int32)).to(self.dev)
        before_b = self.h_buf[:, :i, :].copy()
        before_l = self.h_len[:, :i].copy()
        self.ver.rollback(self.buf, self.lens, i, self.buf[:, i, :], self.lens[:, i].contiguous())
        self._sync()
        if (self.h_len[:, :i] < 0).any():
            raise RuntimeError("rollback reported a buffer length outside [0, cap]")
        changed = (self.h_len[:, :i] != before_l) | (self.h_buf[:, :i, :] != before_b).any(axis=2)
        self.version[:, :i] += changed

    def run(self, tokens):
        """Runs until every stream's final buffer holds `tokens` tokens (or the
        buffers are full); returns the statistics."""
        if tokens + max(self.cfg.gammas) + 2 > self.cfg.cap:
            raise ValueError("cap too small for the requested length")
        self._sync()
        for i in range(self.K):
            self._start(i)
        last = self.K - 1
        room = self.cfg.cap - max(self.cfg.gammas) - 2
        while int(self.h_len[:, last].min()) < tokens and int(self.h_len[:, last].max()) < room:
            self.time = min(self.ends)
            done = [i for i in range(self.K) if self.ends[i] == self.time]
            for i in sorted(done, reverse=True):
                self._apply(i)
            for i in done:
                self._start(i)
        return self.report()

    def final_tokens(self):
        return [list(self.h_buf[s, self.K - 1, :self.h_len[s, self.K - 1]]) for s in range(self.S)]

    def report(self):
        cfg = self.cfg
        g = cfg.gammas[-1]
        st = self.stats[-1]
        live = st.steps - st.discarded
        alpha_w = st.accepted / st.tested if st.tested else 0.0
        tests = st.tested + st.next_tests
        alpha = (st.accepted + st.next_matches) / tests if tests else 0.0
        rho_emp = st.verify_steps / live if live else 0.0
        rho_cf = alpha / (1.0 - alpha ** (g + 1) + alpha) if 0 < alpha < 1 else float(alpha >= 1)
        span = (1.0 - alpha ** (g + 1)) / (1.0 - alpha) if alpha < 1 else g + 1.0
        en_cf = (1.0 - rho_cf) + rho_cf * span
        committed = int(self.h_len[:, -1].sum())
        rate = committed / (self.S * self.time) if self.time else 0.0
        return {
            "time_units": self.time,
            "streams": self.S,
            "final_steps": live,
            "alpha_final": alpha,
            "alpha_final_window_tests": alpha_w,
            "draft_tests": tests,
            "rho_empirical": rho_emp,
            "rho_closed_form": rho_cf,
            "tokens_per_step_empirical": st.emitted / live if live else 0.0,
            "tokens_per_step_eq4": en_cf,
            "verify_steps_full_window": st.full_windows / st.verify_steps if st.verify_steps else 0.0,
            "final_occupancy_hist": list(st.occupancy),
            "tokens_per_time_unit": rate,
            "speedup_vs_autoregressive": rate * cfg.costs[-1],
            "discarded_steps": [s.discarded for s in self.stats],
        }


# Draft noise of HashModels(V=32000, scale 3) giving greedy acceptance of about
# 0.05 / 0.3 / 0.6 / 0.9 between a draft and the noise-free last model.
SIGMA_FOR_GREEDY_ALPHA = {0.05: 3.0, 0.3: 1.3, 0.6: 0.6, 0.9: 0.15}


def sweep(device="cuda", streams=64, tokens=200, V=32000):
    """Two-stage pipelines at the four acceptance levels: verification every
    8 draft steps (windows often partly filled) and every 32 (always full),
    with gamma = 8; plus a three-stage pipeline.  Yields one report per case."""
    for alpha, sig in SIGMA_FOR_GREEDY_ALPHA.items():
        for costs in ((1, 8), (1, 32)):
            cfg = PipeConfig(costs=costs, gammas=(8,), sigmas=(sig, 0.0), V=V, streams=streams,
                             lookahead=32)
            rep = PipeSpecSim(cfg, device=device).run(tokens)
            yield {"stages": 2, "costs": list(costs), "gamma": 8, "target_alpha": alpha, **rep}
    cfg = PipeConfig(costs=(1, 8, 64), gammas=(8, 8), sigmas=(1.3, 0.6, 0.0), V=V, streams=streams,
                     lookahead=32)
    rep = PipeSpecSim(cfg, device=device).run(tokens)
    yield {"stages": 3, "costs": [1, 8, 64], "gamma": 8, **rep}
    # verification dearer than one token: +0.5 time units per window token
    cfg = PipeConfig(costs=(1, 8), gammas=(8,), sigmas=(SIGMA_FOR_GREEDY_ALPHA[0.05], 0.0), V=V,
                     streams=streams, lookahead=32, verify_cost=0.5)
    rep = PipeSpecSim(cfg, device=device).run(tokens)
    yield {"stages": 2, "costs": [1, 8], "gamma": 8, "target_alpha": 0.05, "verify_cost": 0.5, **rep}


if __name__ == "__main__":
    import json
    import sys
    for r in sweep(streams=int(sys.argv[1]) if len(sys.argv) > 1 else 64):
        print(json.dumps(r), flush=True)
