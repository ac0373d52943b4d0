"""Pins of oracle.lmhead_logits / verify_window_lmhead (logits from hidden
states through an unembedding, then the window).

* One-hot unembedding rows (row k of W is e_k): the logits are the hidden
  values themselves, so the result equals oracle.verify_window on them.
* Brute force: a pure-Python triple loop on a tiny case gives the same logits.
* Exact rescaling: hidden * 2^a with W * 2^-a leaves every output unchanged.
* Vocabulary permutation: permuting W's rows and mapping the draft tokens
  through the same permutation permutes the emitted tokens.
"""
import numpy as np
import pytest

import oracle


def _case(rng, gamma=4, H=16, V=12):
    Ht = rng.normal(0, 1, (gamma + 1, H))
    Wt = rng.normal(0, 0.6, (V, H))
    Hd = Ht[:gamma] + rng.normal(0, 0.3, (gamma, H))
    Wd = Wt + rng.normal(0, 0.1, (V, H))
    D = oracle.lmhead_logits(Hd, Wd)
    toks = [int(rng.choice(V, p=oracle.softmax(D[i]))) for i in range(gamma)]
    return Ht, Wt, Hd, Wd, toks


def test_one_hot_unembedding_is_the_window_on_hidden_values():
    rng = np.random.default_rng(1)
    gamma, V = 5, 9
    T = rng.normal(0, 2, (gamma + 1, V))
    D = T[:gamma] + rng.normal(0, 0.5, (gamma, V))
    E = np.eye(V)
    toks = [int(rng.integers(V)) for _ in range(gamma)]
    for seq in range(20):
        u, v = oracle.window_uniforms(3, 0, seq, 0, gamma)
        a = oracle.verify_window_lmhead(T, E, D, E, toks, gamma, u, v)
        b = oracle.verify_window(T, D, toks, gamma, u, v)
        assert a["n"] == b["n"] and a["out"] == b["out"]
        assert np.allclose(a["P"], b["P"], rtol=1e-15) and np.allclose(a["Q"], b["Q"], rtol=1e-15)


def test_brute_force_dot_products():
    rng = np.random.default_rng(2)
    Hm = rng.normal(0, 1, (3, 5))
    W = rng.normal(0, 1, (4, 5))
    L = oracle.lmhead_logits(Hm, W)
    for r in range(3):
        for k in range(4):
            acc = 0.0
            for h in range(5):
                acc += float(Hm[r, h]) * float(W[k, h])
            assert L[r, k] == pytest.approx(acc, rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_exact_rescaling_and_vocabulary_permutation(seed):
    rng = np.random.default_rng(seed)
    Ht, Wt, Hd, Wd, toks = _case(rng)
    gamma, V = len(toks), Wt.shape[0]
    perm = rng.permutation(V)          # new row j holds old token perm[j]
    inv = np.argsort(perm)             # old token k sits at new row inv[k]
    for s in range(10):
        u, v = oracle.window_uniforms(seed, 1, s, 7, gamma)
        a = oracle.verify_window_lmhead(Ht, Wt, Hd, Wd, toks, gamma, u, v)
        b = oracle.verify_window_lmhead(Ht * 4.0, Wt * 0.25, Hd * 0.5, Wd * 2.0, toks, gamma, u, v)
        assert a["n"] == b["n"] and a["out"] == b["out"]
        c = oracle.verify_window_lmhead(Ht, Wt[perm], Hd, Wd[perm], [int(inv[t]) for t in toks], gamma, u, v)
        assert c["n"] == a["n"]
        assert c["out"][:a["n"]] == [int(inv[t]) for t in a["out"][:a["n"]]]
        assert np.allclose(c["P"], a["P"]) and np.allclose(c["Q"], a["Q"])
