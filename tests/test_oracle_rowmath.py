"""Pins of the oracle's per-row arithmetic: decoding, softmax, argmax and the
inverse-CDF sampler, against libraries and brute force."""

import numpy as np
import pytest
import scipy.special
import torch

from oracle import decode, softmax, first_argmax, inverse_cdf

GRID = 2 ** 24


def test_decode_bf16_matches_torch_conversion():
    x = torch.randn(4096, dtype=torch.float32) * 30
    x[:8] = torch.tensor([0.0, -0.0, float("-inf"), 1e-38, -3e38, 1.0, -1.0, 65504.0])
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    got = decode(bits, "bf16")
    want = b.to(torch.float64).numpy()
    assert np.array_equal(got, want)
    assert np.signbit(got[1])


def test_decode_f16_and_f32():
    x = torch.randn(4096, dtype=torch.float32) * 100
    h = x.to(torch.float16)
    assert np.array_equal(decode(h.view(torch.int16).numpy().view(np.uint16), "f16"),
                          h.to(torch.float64).numpy())
    assert np.array_equal(decode(x.numpy(), "f32"), x.numpy().astype(np.float64))
    with pytest.raises(ValueError):
        decode(x.numpy(), "fp8")


def test_softmax_matches_scipy(np_rng):
    for V in (8, 1000, 128256):
        x = np_rng.normal(0, 3, V)
        x[np_rng.integers(0, V, V // 10)] = -np.inf
        p = softmax(x)
        want = scipy.special.softmax(x)
        assert np.allclose(p, want, rtol=1e-12, atol=0)
        fin = np.isfinite(x)
        assert np.all(p[~fin] == 0)
        # log p_k = x_k - logsumexp(x)
        lse = scipy.special.logsumexp(x[fin])
        assert np.allclose(np.log(p[fin]), x[fin] - lse, rtol=0, atol=1e-12)


def test_softmax_rejects_rows_without_finite_logit():
    with pytest.raises(ValueError):
        softmax(np.full(4, -np.inf))


def test_first_argmax_on_tie_laden_bf16_rows(np_rng):
    ties = 0
    for _ in range(200):
        V = int(np_rng.integers(2, 3000))
        x = torch.tensor(np.round(np_rng.normal(0, 2, V) * 2) / 2, dtype=torch.bfloat16)
        row = decode(x.view(torch.int16).numpy().view(np.uint16), "bf16")
        a = first_argmax(row)
        assert a == int(np.argmax(row))
        assert a == min(k for k in range(V) if row[k] == row.max())  # brute force
        ties += int((row == row.max()).sum() > 1)
    assert ties > 20


def test_first_argmax_signed_zero():
    assert first_argmax(np.array([-1.0, -0.0, 0.0, -2.0])) == 1
    assert first_argmax(np.array([-np.inf, -np.inf, -5.0])) == 2


def _scan(w, tau):
    """Brute-force linear scan: smallest k with running sum > tau."""
    s = 0.0
    for k, wk in enumerate(w):
        s += wk
        if s > tau:
            return k
    return None


def test_inverse_cdf_matches_linear_scan(np_rng):
    for _ in range(300):
        V = int(np_rng.integers(1, 50))
        w = np_rng.uniform(0, 1, V) * (np_rng.uniform(0, 1, V) > 0.3)
        if w.sum() == 0:
            w[int(np_rng.integers(0, V))] = 0.5
        v = float(np_rng.integers(0, GRID)) / GRID
        k, info = inverse_cdf(w, v)
        want = _scan(w, v * w.cumsum()[-1])
        if want is None:
            want = int(np.flatnonzero(w > 0)[-1])
        assert k == want
        assert w[k] > 0  # zero-weight tokens are never drawn
        assert info["C_lo"] <= info["tau"] < info["C_hi"] or k == int(np.flatnonzero(w > 0)[-1])


def test_inverse_cdf_bin_widths_on_the_uniform_grid():
    w = np.array([0.1, 0.0, 0.25, 0.05, 0.0, 0.3, 0.2, 0.1])
    Z = w.sum()
    # smallest grid index whose draw exceeds token t, found by bisection
    counts = []
    prev = 0
    for t in range(len(w)):
        lo, hi = 0, GRID
        while lo < hi:
            mid = (lo + hi) // 2
            if inverse_cdf(w, mid / GRID)[0] > t:
                hi = mid
            else:
                lo = mid + 1
        counts.append(lo - prev)
        prev = lo
    counts[-1] += GRID - prev
    assert sum(counts) == GRID
    law = np.array(counts) / GRID
    assert np.allclose(law, w / Z, atol=2.0 / GRID)


def test_inverse_cdf_all_zero_and_single_mass():
    assert inverse_cdf(np.zeros(5), 0.3) == (None, None)
    w = np.zeros(9)
    w[6] = 1e-300
    for v in (0.0, 0.5, 1 - 2 ** -24):
        assert inverse_cdf(w, v)[0] == 6
