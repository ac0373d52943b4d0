"""Chi-square pin of the fused LM-head window (sv_verify_window_lmhead) at
V = 32000 (the LLaMA-2 vocabulary), gamma = 1: 10^5 windows, 100 calls of 1000
sequences, every sequence with the same hidden states and unembeddings but its
own sequence id (so its own Philox uniforms) and its own draft token drawn from
the draft softmax.

Speculative sampling is lossless (CLaSp review, "Assumptions & free
parameters"): the first emitted token follows p_0, and the replacement drawn at
a rejection of the draft follows the renormalised residual max(0, p_0 - q_0).
Here p_0 and q_0 come from the logits of the bf16 hidden states against the
bf16 unembeddings (oracle.lmhead_logits, float64), which the library forms on
the matrix cores in float32.  Bins and threshold (10^-3) as in the oracle's pin
at this size (test_oracle_chi2_large_vocab.py).  Power: the first tokens reject
q_0 and the replacements reject p_0."""
import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

import oracle
import draft_token_verification_06_amd as sv
from test_oracle_chi2_large_vocab import THRESHOLD, _bins, _pvalue

pytestmark = pytest.mark.gpu
DEV = "cuda"
V, GAMMA = 32000, 1
CALLS, B = 100, 1000
HT, HD = 128, 64


def _inputs():
    """One target hidden pair (rows 0, 1) and one draft hidden row, bf16, with
    logits of spread about 2; the draft reads the target's first HD hidden
    entries plus noise against a rescaled slice of the target's unembedding."""
    rng = np.random.default_rng(4321)
    h_t = rng.normal(0.0, 1.0, (GAMMA + 1, HT))
    w_t = rng.normal(0.0, 2.0 / np.sqrt(HT), (V, HT))
    h_d = h_t[:GAMMA, :HD] + rng.normal(0.0, 0.5, (GAMMA, HD))
    w_d = w_t[:, :HD] * np.sqrt(HT / HD)
    return [torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (h_t, w_t, h_d, w_d)]


def test_gpu_lmhead_sampling_law_at_v32000():
    print("GPU LM-head chi-square: 100 calls x 1000 windows, V=32000", flush=True)
    h_t, w_t, h_d, w_d = _inputs()
    T = oracle.lmhead_logits(h_t.float().numpy(), w_t.float().numpy())
    D = oracle.lmhead_logits(h_d.float().numpy(), w_d.float().numpy())
    p0, q0 = sp_softmax(T[0]), sp_softmax(D[0])
    resid = np.maximum(p0 - q0, 0.0)
    resid /= resid.sum()
    cq = np.cumsum(q0)
    ht = h_t.to(DEV)[None].expand(B, GAMMA + 1, HT).contiguous()
    hd = h_d.to(DEV)[None].expand(B, GAMMA, HD).contiguous()
    wt, wd = w_t.to(DEV).contiguous(), w_d.to(DEV).contiguous()
    ws = sv.workspace(sv.SV_OP_LMHEAD, B, GAMMA, V, torch.bfloat16, DEV)
    rng = np.random.default_rng(78)
    n_all, out_all = [], []
    for c in range(CALLS):
        u = rng.random(B)
        toks = np.minimum(V - 1, np.searchsorted(cq, u * cq[-1], side="right")).astype(np.int32)[:, None]
        sid = torch.arange(c * B, (c + 1) * B, dtype=torch.int64, device=DEV)
        res = sv.verify_window_lmhead(ht, wt, hd, wd, torch.from_numpy(toks).to(DEV), seed=6, seq_ids=sid,
                                      ws=ws)
        n_all.append(res.n_accepted.cpu().numpy())
        out_all.append(res.out_tokens.cpu().numpy())
    n = np.concatenate(n_all)
    out = np.concatenate(out_all)
    assert n.min() >= 0 and n.max() <= GAMMA
    first = out[:, 0]
    repl = first[n == 0]
    b0, br = _bins(p0), _bins(resid)
    pv = {"first": _pvalue(first, p0, b0), "replacement": _pvalue(repl, resid, br)}
    power = {"first vs q0": _pvalue(first, q0, b0), "replacement vs p0": _pvalue(repl, p0, br)}
    print("accepted", int((n == 1).sum()), "of", len(n), "p-values", pv, "power", power, flush=True)
    # both branches occur often
    assert len(n) // 10 < (n == 1).sum() < len(n) - len(n) // 10
    assert min(pv.values()) > THRESHOLD
    assert max(power.values()) < 1e-6
