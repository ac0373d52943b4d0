"""Pins of the oracle's per-stage rollback and the three-stage hierarchy
(PipeSpec review, "What carries the argument": each stage appends the
longest matching prefix and on a mismatch all earlier stages roll their
buffers back to the last verified token).

* Post-conditions on random small buffers: every earlier buffer starts with
  the verified sequence, later buffers are untouched, a consistent buffer at
  least as long is kept, anything else ends exactly at the verified length.
* Brute force: a second, independent statement of the same rule.
* Greedy hierarchy: every emitted token equals the final model's argmax.
* Stochastic hierarchy: the first final token follows softmax(final row 0)
  (losslessness applied twice, CLaSp review, "Assumptions & free parameters").
"""

import numpy as np
from scipy.stats import chisquare

from oracle import rollback, hierarchy_three_stage, softmax, first_argmax, window_uniforms


def _random_case(rng, K, cap):
    L = int(rng.integers(0, cap + 1))
    ver = [int(x) for x in rng.integers(0, 4, L)]
    bufs, lens = [], []
    for j in range(K):
        lj = int(rng.integers(0, cap + 1))
        b = [int(x) for x in rng.integers(0, 4, cap)]
        if rng.uniform() < 0.5:  # often agree with the verified prefix
            agree = int(rng.integers(0, min(lj, L) + 1))
            b[:agree] = ver[:agree]
        bufs.append(b)
        lens.append(lj)
    return bufs, lens, ver


def test_rollback_postconditions_and_brute_force():
    rng = np.random.default_rng(61)
    for trial in range(3000):
        K, cap = int(rng.integers(2, 5)), int(rng.integers(1, 9))
        stage = int(rng.integers(1, K))
        bufs, lens, ver = _random_case(rng, K, cap)
        nb, nl = rollback(bufs, lens, stage, ver)
        L = len(ver)
        for j in range(K):
            if j >= stage:
                assert nb[j] == bufs[j] and nl[j] == lens[j]
                continue
            assert nb[j][:L] == ver and nl[j] >= L
            kept = lens[j] >= L and bufs[j][:L] == ver
            # brute force: kept buffers are unchanged, others end at L with the
            # old contents only before the first divergence and after L
            if kept:
                assert nb[j] == bufs[j] and nl[j] == lens[j]
            else:
                assert nl[j] == L
                assert nb[j][L:] == bufs[j][L:]
            assert len(nb[j]) == cap


def test_rollback_examples():
    # diverged at 2: truncate and copy the verified tail
    b, l = rollback([[5, 6, 7, 8, 0], [1, 1, 1, 1, 1]], [4, 1], 1, [5, 6, 9])
    assert b[0] == [5, 6, 9, 8, 0] and l == [3, 1]
    # consistent and longer: kept
    b, l = rollback([[5, 6, 7, 8, 0]], [4], 1, [5, 6])
    assert b[0] == [5, 6, 7, 8, 0] and l == [4]
    # consistent and shorter: extended
    b, l = rollback([[5, 6, 0, 0, 0]], [2], 1, [5, 6, 7, 1])
    assert b[0] == [5, 6, 7, 1, 0] and l == [4]
    # empty verified sequence keeps everything
    b, l = rollback([[3, 3]], [2], 1, [])
    assert b[0] == [3, 3] and l == [2]


def test_greedy_hierarchy_emits_final_argmax_sequence():
    rng = np.random.default_rng(67)
    g1, g2, V = 8, 4, 10
    for s in range(300):
        F = np.round(rng.normal(0, 1, (g1 + 1, V)) * 2) / 2
        S1 = F + (rng.normal(0, 0.4, (g1 + 1, V)) if s % 3 else 0)
        S0 = F[:g1] + rng.normal(0, 1.0, (g1, V))
        o0 = [first_argmax(S0[i]) for i in range(g1)]
        r = hierarchy_three_stage(F, S1, S0, o0, g1, g2, "greedy", None, None)
        O2 = r["O2"]
        assert O2 == [first_argmax(F[i]) for i in range(len(O2))]
        L2 = len(O2)
        for j in range(2):
            assert r["buffers"][j][:L2] == O2 and r["lengths"][j] >= L2
        L1 = len(r["O1"])
        assert r["O1"] == [first_argmax(S1[i]) for i in range(L1)]


def test_stochastic_hierarchy_first_token_follows_final_model():
    rng = np.random.default_rng(71)
    g1, g2, V, N = 3, 2, 8, 12000
    F = rng.normal(0, 1, (g1 + 1, V))
    S1 = F + rng.normal(0, 0.5, (g1 + 1, V))
    S0 = F[:g1] + rng.normal(0, 1.0, (g1, V))
    q0 = [softmax(S0[i]) for i in range(g1)]
    first = []
    for s in range(N):
        o0 = [int(rng.choice(V, p=q0[i])) for i in range(g1)]
        uv1 = window_uniforms(0, 1, s, 0, g1)
        uv2 = window_uniforms(0, 2, s, 0, g2)
        r = hierarchy_three_stage(F, S1, S0, o0, g1, g2, "stochastic", uv1, uv2)
        first.append(r["O2"][0])
    counts = np.bincount(first, minlength=V)
    assert chisquare(counts, N * softmax(F[0])).pvalue > 1e-3
    assert chisquare(counts, N * softmax(S1[0])).pvalue < 1e-3  # power
