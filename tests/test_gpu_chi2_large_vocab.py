"""Chi-square pins of the HIP library's own sampling law at V = 32000 (the
LLaMA-2 vocabulary), gamma = 2, float32 logits: 10^5 windows, 100 calls of
1000 sequences, each sequence with its own sequence id (so its own Philox
uniforms) and its own draft tokens drawn from the draft softmax.

Speculative sampling is lossless (CLaSp review, "Assumptions & free
parameters"): the first emitted token follows p_0, the second, on windows that
accepted draft 0, follows p_1, the bonus after a full window follows p_2, and
the replacement drawn at a rejection of draft 0 follows the renormalised
residual max(0, p_0 - q_0).  The expected laws come from scipy's softmax of the
float32 rows the library reads; bins and threshold (10^-3) as in the oracle's
pin at this size (test_oracle_chi2_large_vocab.py).  Power: the first tokens
reject q_0 and the replacements reject p_0.  The second test draws the same
10^5 windows as 2000 calls of 50 sequences, through the split draw (several
workgroups per sequence's sampling pass, the last to finish searching); the
third draws 10^6 windows on bf16 logits."""
import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

import draft_token_verification_06_amd as sv
from test_oracle_chi2_large_vocab import THRESHOLD, _bins, _pvalue

pytestmark = pytest.mark.gpu
DEV = "cuda"
V, GAMMA = 32000, 2
CALLS, B = 100, 1000


def _rows():
    rng = np.random.default_rng(32000)
    T = rng.normal(0.0, 2.0, (GAMMA + 1, V)).astype(np.float32)
    D = (T[:GAMMA].astype(np.float64) + rng.normal(0.0, 0.5, (GAMMA, V))).astype(np.float32)
    return T, D


def _sampling_law(B, calls, draw_seed, philox_seed, dtype=torch.float32):
    """10^5 windows as `calls` calls of B sequences, logits stored as `dtype`;
    the expected laws come from the stored values; every law asserted."""
    T, D = _rows()
    Tt, Dt = torch.from_numpy(T).to(dtype), torch.from_numpy(D).to(dtype)
    Tf, Df = Tt.double().numpy(), Dt.double().numpy()
    p = [sp_softmax(Tf[i]) for i in range(GAMMA + 1)]
    q = [sp_softmax(Df[i]) for i in range(GAMMA)]
    cq = [np.cumsum(x) for x in q]
    target = Tt.to(DEV)[None].expand(B, GAMMA + 1, V).contiguous()
    draft = Dt.to(DEV)[None].expand(B, GAMMA, V).contiguous()
    ws = sv.workspace(sv.SV_OP_WINDOW, B, GAMMA, V, dtype, DEV)
    rng = np.random.default_rng(draw_seed)
    n_all, out_all = [], []
    for c in range(calls):
        u = rng.random((B, GAMMA))
        toks = np.stack([np.minimum(V - 1, np.searchsorted(cq[i], u[:, i] * cq[i][-1], side="right"))
                         for i in range(GAMMA)], axis=1).astype(np.int32)
        sid = torch.arange(c * B, (c + 1) * B, dtype=torch.int64, device=DEV)
        res = sv.verify_window(target, draft, torch.from_numpy(toks).to(DEV), seed=philox_seed, seq_ids=sid,
                               ws=ws)
        n_all.append(res.n_accepted.cpu().numpy())
        out_all.append(res.out_tokens.cpu().numpy())
    n = np.concatenate(n_all)
    out = np.concatenate(out_all)
    assert n.min() >= 0 and n.max() <= GAMMA
    first = out[:, 0]
    b0 = _bins(p[0])
    pv = {"first": _pvalue(first, p[0], b0),
          "second": _pvalue(out[n >= 1, 1], p[1], _bins(p[1])),
          "bonus": _pvalue(out[n == GAMMA, GAMMA], p[GAMMA], _bins(p[GAMMA]))}
    r = np.maximum(0.0, p[0] - q[0])
    br = _bins(r)
    pv["replacement"] = _pvalue(out[n == 0, 0], r, br)
    power = {"first_vs_q0": _pvalue(first, q[0], b0), "replacement_vs_p0": _pvalue(out[n == 0, 0], p[0], br)}
    print("p-values", pv, "power", power, "windows", len(n), "n=0/1/2", np.bincount(n, minlength=3),
          flush=True)
    assert (n >= 1).sum() > len(n) // 2 and (n == GAMMA).sum() > len(n) // 3 and (n == 0).sum() > len(n) // 10
    for k, v in pv.items():
        assert v > THRESHOLD, (k, v)
    for k, v in power.items():
        assert v < 1e-6, (k, v)


def test_gpu_sampling_law_at_v32000():
    print("GPU chi-square: 100 calls x 1000 windows, V=32000", flush=True)
    _sampling_law(B, CALLS, 77, 5)


def test_gpu_sampling_law_split_draw_at_v32000():
    """The same laws through the split draw: at 50 sequences per call each
    sequence's sampling pass is shared by 6 workgroups (float32 rows of
    V = 32000 are 8 chunks) and the last to finish searches; 2000 calls."""
    print("GPU chi-square, split draw: 2000 calls x 50 windows, V=32000", flush=True)
    _sampling_law(50, 2000, 79, 7)


def test_gpu_sampling_law_bf16_rows_at_v32000():
    """The same laws on bf16 logits (the benchmark's storage type: its decode
    and 8-element vectors in the sampling pass) over 10^6 windows, 1000 calls of
    1000 sequences: at this count a bin's probability is checked to about 1%
    of itself."""
    print("GPU chi-square, bf16 rows: 1000 calls x 1000 windows, V=32000", flush=True)
    _sampling_law(B, 10 * CALLS, 81, 9, dtype=torch.bfloat16)
