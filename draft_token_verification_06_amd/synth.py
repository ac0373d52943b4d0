"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the logits dtype; it
holds none of the verification arithmetic (no softmax, no accept rule, no
sampling from residuals).  Draft tokens are drawn from softmax(draft logits)
with the Gumbel-max construction: argmax_k (d_k + G_k) with G_k standard
Gumbel noise, evaluated in float64 on the already-rounded draft logits, so the
draft law is exactly the distribution the verifier sees.

Workload shapes follow the models the pages name (vocabularies 32000 for
LLaMA-2, 50257 for GPT-2-L, 128256 for LLaMA-3/3.1; window 8 as the
speculative-decoding lookahead in the PipeSpec review):

* window_config1 -- B=1, gamma=4, V=32000, fp32, target N(0, 2^2), draft =
  target + N(0, 0.5^2).
* window_batch   -- B sequences, target N(0, sd^2) plus a boost on one random
  token per row, draft = target + N(0, sigma^2), any dtype; the B=8 and B=256
  gamma=8 V=128256 bf16 workloads use it (sigma chosen per acceptance rate).
* tree_config3   -- B=4, tree with branching (4, 3, 2) (41 nodes, BFS order),
  V=50257, fp16; children drawn i.i.d. from softmax(draft of the parent).
* hierarchy_config4 -- 64 streams, V=128256, bf16, final-stage logits
  N(0, 3^2), stage-1 = final + N(0, 0.3^2), stage-0 = final + N(0, 1^2).
* alpha_exact_window -- probabilities built so that sum_k min(p_k, q_k) is
  exactly alpha at every position (float64, small vocabularies).

All generators are deterministic given (seed, device); CPU and GPU draws differ,
so a comparison always copies the generated bits to the host for the oracle.
"""

import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# Draft-noise standard deviation giving a mean per-token acceptance rate alpha
# on the gamma=8, V=128256 bf16 workload (target N(0, 3^2) + 6 on one token
# per row).  Calibrated with the float64 oracle on this module's own draws;
# tests/test_synth.py re-checks the mapping on a sample.
SIGMA_FOR_ALPHA = {0.05: 4.40, 0.3: 2.12, 0.6: 1.06, 0.9: 0.255}


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gumbel_max_tokens(draft, g, chunk_rows=64):
    """Draw one token per row from softmax(draft) by the Gumbel-max trick.

    draft: (..., V) tensor of the rounded draft logits.  Returns int32 (...).
    """
    shape = draft.shape[:-1]
    V = draft.shape[-1]
    flat = draft.reshape(-1, V)
    out = torch.empty(flat.shape[0], dtype=torch.int32, device=draft.device)
    tiny = torch.finfo(torch.float64).tiny
    for r0 in range(0, flat.shape[0], chunk_rows):
        rows = flat[r0 : r0 + chunk_rows].to(torch.float64)
        U = torch.rand(rows.shape, generator=g, dtype=torch.float64, device=draft.device)
        G = -torch.log(-torch.log(U.clamp_min(tiny)))
        out[r0 : r0 + chunk_rows] = torch.argmax(rows + G, dim=-1).to(torch.int32)
    return out.reshape(shape)


def _normal(shape, sd, g, device):
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device) * sd


def window_batch(B, gamma, V, dtype="bf16", target_sd=3.0, boost=6.0, sigma=1.0,
                 seed=0, device="cpu"):
    """Batched window: target (B, gamma+1, V), draft (B, gamma, V), tokens."""
    g = generator(seed, device)
    tdt = DTYPES[dtype]
    T = _normal((B, gamma + 1, V), target_sd, g, device)
    if boost:
        idx = torch.randint(0, V, (B, gamma + 1, 1), generator=g, device=device)
        T.scatter_add_(2, idx, torch.full((B, gamma + 1, 1), float(boost), device=device))
    target = T.to(tdt)
    D = target[:, :gamma].to(torch.float32) + _normal((B, gamma, V), sigma, g, device)
    del T
    draft = D.to(tdt)
    del D
    tokens = gumbel_max_tokens(draft, g)
    return {"target": target, "draft": draft, "tokens": tokens, "dtype": dtype,
            "gamma": gamma, "V": V, "B": B}


def window_config1(seed=1001, device="cpu"):
    """B=1, gamma=4, V=32000, fp32: target N(0, 2^2), draft = target + N(0, 0.5^2)."""
    return window_batch(1, 4, 32000, dtype="f32", target_sd=2.0, boost=0.0,
                        sigma=0.5, seed=seed, device=device)


def window_config5(alpha, B=256, seed=1005, device="cpu"):
    """B=256, gamma=8, V=128256, bf16, draft noise set for acceptance alpha."""
    return window_batch(B, 8, 128256, dtype="bf16", target_sd=3.0, boost=6.0,
                        sigma=SIGMA_FOR_ALPHA[alpha], seed=seed, device=device)


def bfs_tree(branching):
    """Parent array of a complete tree in BFS order, e.g. (4, 3, 2) -> 41 nodes."""
    parent = [-1]
    level = [0]
    for b in branching:
        nxt = []
        for w in level:
            for _ in range(b):
                parent.append(w)
                nxt.append(len(parent) - 1)
        level = nxt
    return parent


def tree_batch(B, parent, V, dtype="f16", target_sd=2.0, sigma=0.5, seed=1003,
               device="cpu"):
    """Tree batch: target/draft (B, N, V); node tokens drawn i.i.d. from
    softmax(rounded draft row of the parent), with replacement."""
    g = generator(seed, device)
    N = len(parent)
    tdt = DTYPES[dtype]
    T = _normal((B, N, V), target_sd, g, device)
    target = T.to(tdt)
    draft = (target.to(torch.float32) + _normal((B, N, V), sigma, g, device)).to(tdt)
    del T
    par = torch.tensor([max(p, 0) for p in parent], device=device)
    parent_rows = draft[:, par]  # (B, N, V): row of each node's parent
    tokens = gumbel_max_tokens(parent_rows, g)
    tokens[:, 0] = 0
    return {"target": target, "draft": draft, "tokens": tokens, "parent": list(parent),
            "dtype": dtype, "V": V, "B": B}


def tree_config3(seed=1003, device="cpu"):
    return tree_batch(4, bfs_tree((4, 3, 2)), 50257, seed=seed, device=device)


def hierarchy_config4(S=64, V=128256, gamma1=8, mode="greedy", seed=1004, device="cpu",
                      dtype="bf16"):
    """PipeSpec-shaped three-stage hierarchy inputs.

    F (S, gamma1+1, V) final model, S1 (S, gamma1+1, V) = F + N(0, 0.3^2),
    S0 (S, gamma1, V) = F + N(0, 1^2); o0 = stage-0 drafts (argmax of S0 rows
    for greedy, draws from softmax(S0 rows) otherwise)."""
    g = generator(seed, device)
    tdt = DTYPES[dtype]
    F32 = _normal((S, gamma1 + 1, V), 3.0, g, device)
    F = F32.to(tdt)
    S1 = (F.to(torch.float32) + _normal((S, gamma1 + 1, V), 0.3, g, device)).to(tdt)
    S0 = (F[:, :gamma1].to(torch.float32) + _normal((S, gamma1, V), 1.0, g, device)).to(tdt)
    del F32
    if mode == "greedy":
        o0 = torch.argmax(S0.to(torch.float32), dim=-1).to(torch.int32)
    else:
        o0 = gumbel_max_tokens(S0, g)
    return {"F": F, "S1": S1, "S0": S0, "o0": o0, "dtype": dtype, "V": V, "S": S,
            "gamma1": gamma1}


def lmhead_batch(B, gamma, V, Ht, Hd, logit_sd=3.0, noise=0.5, seed=0, device="cpu"):
    """Hidden states and unembeddings (bf16) for the LM-head window.

    Target: hidden rows ~ N(0, 1) of width Ht, unembedding rows ~ N(0, sd^2 / Ht)
    (logits of standard deviation ~logit_sd).  Draft (width Hd <= Ht): its
    unembedding is the target's first Hd columns rescaled by sqrt(Ht / Hd), its
    hidden rows the target's first Hd entries plus N(0, noise^2), so draft and
    target logits are correlated.  Draft tokens are drawn from the draft's own
    logits (computed here in float32 from the rounded inputs)."""
    if Hd > Ht:
        raise ValueError("the draft's hidden width must not exceed the target's")
    g = generator(seed, device)
    h_t = _normal((B, gamma + 1, Ht), 1.0, g, device).to(torch.bfloat16)
    w_t = _normal((V, Ht), logit_sd / Ht ** 0.5, g, device).to(torch.bfloat16)
    h_d = (h_t[:, :gamma, :Hd].to(torch.float32) + _normal((B, gamma, Hd), noise, g, device)
           ).to(torch.bfloat16).contiguous()
    w_d = (w_t[:, :Hd].to(torch.float32) * (Ht / Hd) ** 0.5).to(torch.bfloat16).contiguous()
    D = (h_d.to(torch.float32).reshape(-1, Hd) @ w_d.to(torch.float32).T).reshape(B, gamma, V)
    tokens = gumbel_max_tokens(D, g)
    del D
    return {"h_target": h_t, "w_target": w_t, "h_draft": h_d, "w_draft": w_d, "tokens": tokens,
            "B": B, "gamma": gamma, "V": V, "Ht": Ht, "Hd": Hd}


def alpha_exact_probs(alpha, V, rng):
    """(p, q) with sum_k min(p_k, q_k) == alpha exactly.

    p = alpha*s + (1-alpha)*a and q = alpha*s + (1-alpha)*b where s > 0 on every
    token and a, b are distributions on disjoint halves of the vocabulary."""
    s = rng.uniform(0.5, 1.5, V)
    s /= s.sum()
    half = V // 2
    a = np.zeros(V)
    b = np.zeros(V)
    a[:half] = rng.uniform(0.1, 1.0, half)
    b[half:] = rng.uniform(0.1, 1.0, V - half)
    a /= a.sum()
    b /= b.sum()
    return alpha * s + (1 - alpha) * a, alpha * s + (1 - alpha) * b


def alpha_exact_window(alpha, gamma, V, rng):
    """One window of exact-alpha float64 logits: target (gamma+1, V) and draft
    (gamma, V) as log-probabilities, with draft tokens drawn from q by
    inverse transform on numpy's generator (independent of Philox)."""
    T = np.empty((gamma + 1, V))
    D = np.empty((gamma, V))
    toks = np.empty(gamma, dtype=np.int64)
    for i in range(gamma + 1):
        p, q = alpha_exact_probs(alpha, V, rng)
        T[i] = np.log(p)
        if i < gamma:
            D[i] = np.log(q)
            toks[i] = rng.choice(V, p=q)
    return T, D, toks


def to_host_bits(t):
    """Host numpy copy of a logits tensor in the oracle's input form
    (uint16 bit patterns for bf16/f16, float32 otherwise)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def round_trip_sigma(alpha):
    """Log-normal first guess of the noise sd for acceptance alpha
    (alpha ~ 2*Phi(-sigma/2)), used only as a calibration starting point."""
    lo, hi = 1e-4, 20.0
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        a = math.erfc(mid / 2 / math.sqrt(2))
        lo, hi = (mid, hi) if a > alpha else (lo, mid)
    return 0.5 * (lo + hi)
