"""GPU parity of sv_verify_window_lmhead (LM head on the matrix cores fused
with the window) against oracle.verify_window_lmhead (float64 logits from the
same bf16 hidden states and unembeddings): p(x), q(x) within 1e-5 relative,
n and tokens identical except margin cases (at most one per test); ragged
row and column tiles, partial windows, invalid tokens, caller-chosen uniform
keys, small batches (split draw) and the 8B/1B-shaped workload on sampled
sequences."""
import numpy as np
import pytest
import torch

import oracle
import draft_token_verification_06_amd as sv
from draft_token_verification_06_amd import synth
from gpu_common import check_lmhead, host_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(d, seed, **kw):
    return sv.verify_window_lmhead(d["h_target"], d["w_target"], d["h_draft"], d["w_draft"], d["tokens"],
                                   seed=seed, return_probs=True, **kw)


@pytest.mark.parametrize("B,gamma,V,Ht,Hd", [
    (4, 4, 1000, 128, 64),      # one ragged column tile, rows within one block
    (5, 3, 300, 64, 64),
    (40, 8, 5003, 256, 192),    # several row blocks, odd vocabulary
    (3, 64, 777, 64, 64),       # longest window
])
def test_lmhead_small(B, gamma, V, Ht, Hd):
    print("lmhead", B, gamma, V, Ht, Hd, flush=True)
    d = synth.lmhead_batch(B, gamma, V, Ht, Hd, seed=100 + B, device=DEV)
    res = _run(d, seed=B)
    n, m = check_lmhead(d, res, seed=B)
    assert m <= 1


def test_lmhead_partial_windows_and_invalid_tokens():
    print("lmhead partial/invalid", flush=True)
    B, gamma, V = 12, 6, 2048
    d = synth.lmhead_batch(B, gamma, V, 128, 128, seed=7, device=DEV)
    wl = torch.tensor([0, 1, 2, 3, 4, 5, 6, 6, 6, 6, 0, 3], dtype=torch.int32, device=DEV)
    d["tokens"][8, 2] = V        # inside the window: the sequence is marked
    d["tokens"][11, 5] = -4      # past window_len 3: ignored
    res = _run(d, seed=3, window_len=wl)
    assert res.n_accepted[8].item() == -1 and (res.out_tokens[8] == -1).all()
    rows = [b for b in range(B) if b != 8]
    n, m = check_lmhead(d, res, seed=3, window_len=wl, rows=rows)
    assert m <= 1


@pytest.mark.parametrize("B", [5, 300])
def test_lmhead_caller_keys(B):
    """Uniforms keyed by the caller: random sequence ids and base positions
    and a nonzero tag, drawn through both draw launches (float32 rows of
    V = 9000 are three 16 KB chunks: at B = 5 each sequence's draw is split over
    three workgroups and the last to finish draws; at B = 300 one workgroup
    draws).  Every sequence is checked against the oracle with the same keys."""
    print("lmhead caller keys", B, flush=True)
    gamma, V = 4, 9000
    d = synth.lmhead_batch(B, gamma, V, 128, 64, seed=500 + B, device=DEV)
    rng = np.random.default_rng(77 + B)
    sid = torch.from_numpy(rng.integers(0, 2 ** 40, B).astype(np.int64)).to(DEV)
    bp = torch.from_numpy(rng.integers(0, 10 ** 6, B).astype(np.int64)).to(DEV)
    res = _run(d, seed=9, tag=3, seq_ids=sid, base_pos=bp)
    n, m = check_lmhead(d, res, seed=9, tag=3, seq_ids=sid, base_pos=bp)
    assert n == B and m <= 1
    # the keys matter: the default keys give other decisions somewhere
    plain = _run(d, seed=9)
    assert not torch.equal(plain.out_tokens, res.out_tokens)


def test_lmhead_8b_1b_shape_sampled():
    """B=256, gamma=8, V=128256, Ht=4096, Hd=2048 (the shape of an 8B target
    with a 1B draft); eight sampled sequences against the oracle."""
    print("lmhead full shape", flush=True)
    d = synth.lmhead_batch(256, 8, 128256, 4096, 2048, seed=2024, device=DEV)
    res = _run(d, seed=11)
    n, m = check_lmhead(d, res, seed=11, rows=[0, 31, 64, 100, 127, 128, 200, 255])
    assert m <= 1


def test_lmhead_is_deterministic():
    d = synth.lmhead_batch(16, 8, 4096, 256, 128, seed=5, device=DEV)
    a = _run(d, seed=2)
    b = _run(d, seed=2)
    assert torch.equal(a.n_accepted, b.n_accepted) and torch.equal(a.out_tokens, b.out_tokens)
    assert torch.equal(a.p_draft, b.p_draft) and torch.equal(a.q_draft, b.q_draft)


@pytest.mark.parametrize("k", range(6))
def test_random_lmhead_configuration(k):
    """Random shapes against the oracle: B, gamma, a vocabulary that often
    leaves a ragged last column tile, and hidden widths of one to eight K
    steps (the GEMM's first and last steps load clamped tiles)."""
    rng = np.random.default_rng(9100 + k)
    B = int(rng.choice([1, 3, 17, 40]))
    gamma = int(rng.choice([1, 3, 8, 13]))
    V = int(rng.choice([7, 257, 1000, 4099]))
    Ht = 64 * int(rng.integers(1, 9))
    Hd = 64 * int(rng.integers(1, Ht // 64 + 1))
    seed = int(rng.integers(0, 1000))
    print("lmhead random", k, B, gamma, V, Ht, Hd, flush=True)
    d = synth.lmhead_batch(B, gamma, V, Ht, Hd, seed=seed, device=DEV)
    res = _run(d, seed=seed)
    n, m = check_lmhead(d, res, seed=seed)
    assert m <= 1
