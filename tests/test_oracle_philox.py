"""Pins of the oracle's Philox4x64-10 stream and uniform mapping.

The oracle implements Philox from its published definition; numpy ships an
independent Philox4x64-10 (``numpy.random.Philox``).  numpy advances its
counter by one *before* computing a block, so its first block from counter
state c is the bijection at c + 1 (fixed by the experiment in
test_numpy_counter_convention)."""

import numpy as np
import pytest

from oracle import philox4x64_10, uniform24, window_uniforms, tree_uniforms, tree_meta

M256 = (1 << 256) - 1


def _numpy_block(counter_words, key_words):
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter_words))
    k = int(key_words[0]) | (int(key_words[1]) << 64)
    g = np.random.Philox(counter=(c - 1) & M256, key=k)
    return [int(x) for x in g.random_raw(4)]


def test_numpy_counter_convention():
    g = np.random.Philox(counter=0, key=0)
    first = [int(x) for x in g.random_raw(4)]
    assert list(g.state["state"]["counter"]) == [1, 0, 0, 0]
    assert first == list(philox4x64_10((1, 0, 0, 0), (0, 0)))
    assert first != list(philox4x64_10((0, 0, 0, 0), (0, 0)))


def test_philox_matches_numpy_bit_for_bit():
    rng = np.random.default_rng(2024)
    for trial in range(1200):
        if trial < 200:  # small structured counters as the library uses them
            ctr = (int(rng.integers(0, 1 << 20)), int(rng.integers(0, 1 << 12)),
                   int(rng.integers(0, 64)), 0)
            key = (int(rng.integers(0, 1 << 63)), int(rng.integers(0, 4)))
        else:
            ctr = tuple(int(x) for x in rng.integers(0, 1 << 63, 4, dtype=np.uint64) * 2
                        + rng.integers(0, 2, 4, dtype=np.uint64))
            key = tuple(int(x) for x in rng.integers(0, 1 << 63, 2, dtype=np.uint64) * 2
                        + rng.integers(0, 2, 2, dtype=np.uint64))
        assert list(philox4x64_10(ctr, key)) == _numpy_block(ctr, key), (ctr, key)


def test_philox_carry_into_high_counter_words():
    ctr = ((1 << 64) - 1, (1 << 64) - 1, 5, 0)
    assert list(philox4x64_10(ctr, (7, 9))) == _numpy_block(ctr, (7, 9))


def test_uniform_grid_and_range():
    assert uniform24(0) == 0.0
    assert uniform24((1 << 64) - 1) == 1.0 - 2.0 ** -24
    rng = np.random.default_rng(1)
    for w in rng.integers(0, 1 << 63, 500, dtype=np.uint64):
        u = uniform24(int(w) * 2 + 1)
        assert 0.0 <= u < 1.0
        assert float(np.float32(u)) == u  # exact in float32
        assert (u * 2 ** 24).is_integer()


def test_chain_tree_draws_window_uniforms():
    gamma = 6
    parent = [-1] + list(range(gamma))
    depth, rank, _ = tree_meta(parent)
    u_w, v_w = window_uniforms(3, 1, 17, 40, gamma)
    u_t, v_t = tree_uniforms(3, 1, 17, 40, depth, rank)
    assert u_t[1:] == u_w[:gamma]
    assert v_t == v_w


def test_stages_and_windows_do_not_share_uniforms():
    u1, v1 = window_uniforms(0, 1, 5, 0, 8)
    u2, v2 = window_uniforms(0, 2, 5, 0, 8)
    u3, _ = window_uniforms(0, 1, 5, 9, 8)   # next window after 8 accepted + bonus
    assert not set(u1) & set(u2)
    assert not set(u1) & set(u3)
    assert u1 != v1
