"""Chi-square pins of the oracle's speculative sampling at a realistic
vocabulary: V = 32000 (the LLaMA-2 vocabulary the pages' models use), gamma = 2,
10^5 windows driven by the real Philox uniform stream (seed 0, tag 0, sequence
ids 0..10^5-1).

Speculative sampling is lossless (CLaSp review, "Assumptions & free
parameters"): the first emitted token follows p_0, the second, on windows that
accepted draft 0, follows p_1, and the bonus after a full window follows
p_gamma.  The replacement drawn at a rejection of draft 0 follows the
renormalised residual max(0, p_0 - q_0).  Each law is tested on 100 bins that
are contiguous in token order and hold about equal mass under the law tested
(so a bin is a few hundred tokens, or one heavy token), against a threshold
fixed in advance at 10^-3.  Power: the same statistic rejects q_0 for the
first token and p_0 for the replacement (non-centrality about 2000 on these
rows).  The expected laws come from scipy's softmax, not the oracle's.

Rows: target N(0, 2^2), draft = target + N(0, 0.5^2) (the B=1 gamma=4
V=32000 workload's generator), in float64; draft tokens are drawn from the
draft softmax by inverse CDF with a numpy generator seeded per window, so the
outcome does not depend on how the windows are split over processes.
"""
import multiprocessing
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chisquare

from oracle import verify_window, window_uniforms

pytestmark = pytest.mark.slow

V, GAMMA, N = 32000, 2, 100_000
THRESHOLD = 1e-3


def _rows():
    rng = np.random.default_rng(32000)
    T = rng.normal(0.0, 2.0, (GAMMA + 1, V))
    D = T[:GAMMA] + rng.normal(0.0, 0.5, (GAMMA, V))
    return T, D


def _windows(bounds):
    lo, hi = bounds
    T, D = _rows()
    cq = [np.cumsum(sp_softmax(D[i])) for i in range(GAMMA)]
    out = []
    for s in range(lo, hi):
        rng = np.random.default_rng([7, s])
        toks = [min(V - 1, int(np.searchsorted(c, rng.random() * c[-1], side="right"))) for c in cq]
        u, v = window_uniforms(0, 0, s, 0, GAMMA)
        o = verify_window(T, D, toks, GAMMA, u, v)
        out.append((o["n"], o["out"]))
    return out


@pytest.fixture(scope="module")
def windows():
    procs = max(1, min(8, len(os.sched_getaffinity(0))))
    step = 2500
    chunks = [(lo, min(N, lo + step)) for lo in range(0, N, step)]
    with multiprocessing.get_context("fork").Pool(procs) as pool:
        parts = pool.map(_windows, chunks)
    return [w for part in parts for w in part]


def _bins(w, nb=100):
    """Bin of every token: contiguous in token order, about 1/nb of w's mass each."""
    w = w / w.sum()
    before = np.cumsum(w) - w
    return np.minimum(nb - 1, np.floor(before * nb).astype(np.int64))


def _pvalue(tokens, law, bins):
    """Chi-square p-value of the tokens' bin counts against `law` on `bins`
    (bins with no mass under the binning law are left out)."""
    law = law / law.sum()
    nb = int(bins.max()) + 1
    expect = np.bincount(bins, weights=law, minlength=nb) * len(tokens)
    count = np.bincount(bins[np.asarray(tokens)], minlength=nb).astype(np.float64)
    keep = np.bincount(bins, minlength=nb) > 0
    assert count[~keep].sum() == 0
    return chisquare(count[keep], expect[keep] * count[keep].sum() / expect[keep].sum()).pvalue


def test_first_emitted_token_follows_p0(windows):
    T, D = _rows()
    p0, q0 = sp_softmax(T[0]), sp_softmax(D[0])
    first = [w[1][0] for w in windows]
    assert len(first) == N
    bins = _bins(p0)
    assert _pvalue(first, p0, bins) > THRESHOLD
    assert _pvalue(first, q0, bins) < 1e-6  # power: the draft law is told apart


def test_second_token_after_accepted_draft_follows_p1(windows):
    T, _ = _rows()
    p1 = sp_softmax(T[1])
    second = [w[1][1] for w in windows if w[0] >= 1]
    assert len(second) > N // 2
    assert _pvalue(second, p1, _bins(p1)) > THRESHOLD


def test_bonus_after_full_window_follows_p_gamma(windows):
    T, _ = _rows()
    pg = sp_softmax(T[GAMMA])
    bonus = [w[1][GAMMA] for w in windows if w[0] == GAMMA]
    assert len(bonus) > N // 3
    assert _pvalue(bonus, pg, _bins(pg)) > THRESHOLD


def test_replacement_after_first_rejection_follows_residual(windows):
    T, D = _rows()
    p0, q0 = sp_softmax(T[0]), sp_softmax(D[0])
    r = np.maximum(0.0, p0 - q0)
    repl = [w[1][0] for w in windows if w[0] == 0]
    assert len(repl) > N // 10
    bins = _bins(r)
    assert _pvalue(repl, r, bins) > THRESHOLD
    assert _pvalue(repl, p0, bins) < 1e-6  # power: a draw from p instead is told apart
