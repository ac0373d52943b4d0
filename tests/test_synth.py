"""Checks of the seeded input generators (no verification arithmetic lives
there; the float64 oracle measures what they produce)."""

import numpy as np
import pytest
import torch
from scipy.stats import chisquare

from draft_token_verification_06_amd import synth
from oracle import decode, softmax


def test_generators_are_deterministic():
    a = synth.window_batch(2, 3, 1000, "bf16", sigma=0.5, seed=5)
    b = synth.window_batch(2, 3, 1000, "bf16", sigma=0.5, seed=5)
    assert torch.equal(a["target"].view(torch.int16), b["target"].view(torch.int16))
    assert torch.equal(a["tokens"], b["tokens"])
    assert a["target"].shape == (2, 4, 1000) and a["draft"].shape == (2, 3, 1000)
    assert a["tokens"].dtype == torch.int32


def test_gumbel_max_draws_follow_softmax():
    V, N = 8, 40000
    logits = torch.tensor(np.random.default_rng(1).normal(0, 1, V), dtype=torch.float32)
    toks = synth.gumbel_max_tokens(logits.expand(N, V).contiguous(), synth.generator(3))
    counts = np.bincount(toks.numpy(), minlength=V)
    p = softmax(logits.double().numpy())
    assert chisquare(counts, N * p).pvalue > 1e-3


def test_alpha_exact_probs_have_overlap_alpha():
    rng = np.random.default_rng(2)
    for alpha in (0.0, 0.05, 0.5, 0.9, 1.0):
        p, q = synth.alpha_exact_probs(alpha, 16, rng)
        assert abs(p.sum() - 1) < 1e-12 and abs(q.sum() - 1) < 1e-12
        assert abs(np.minimum(p, q).sum() - alpha) < 1e-12


def test_bfs_tree_shape():
    par = synth.bfs_tree((4, 3, 2))
    assert len(par) == 41 and par[0] == -1 and all(0 <= par[v] < v for v in range(1, 41))


@pytest.mark.parametrize("alpha", sorted(synth.SIGMA_FOR_ALPHA))
def test_noise_calibration_gives_the_named_acceptance(alpha):
    d = synth.window_config5(alpha, B=2, seed=77)
    T = decode(synth.to_host_bits(d["target"]), "bf16")
    D = decode(synth.to_host_bits(d["draft"]), "bf16")
    a = [np.minimum(softmax(T[b, i]), softmax(D[b, i])).sum() for b in range(2) for i in range(8)]
    assert abs(np.mean(a) - alpha) < 0.035
