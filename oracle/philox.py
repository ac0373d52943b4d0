"""Counter-based uniforms for the oracle (test infrastructure only).

The pages fix no random-number generator.  The library keys its uniforms on a
counter-based Philox stream indexed by (seed, sequence, position); this module
is the oracle's own implementation of that stream, written from the published
definition of Philox4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): two 64x64->128-bit
multiplies per round, a Weyl-sequence key schedule, 10 rounds.

Key    = (seed, tag)          -- tag separates stages of a hierarchy.
Counter= (seq_id, pos, rank, 0)
  pos  = absolute position of the token being decided / produced
         (base_pos + 1 + i for draft i of a window; base_pos + depth for a
         tree node; base_pos + depth(d) + 1 for the token sampled after d),
  rank = index of a tree node among the nodes at its depth (0 for windows).
Word 0 -> the accept uniform u of the draft token at (pos, rank).
Word 1 -> the sampling uniform v of the token produced at (pos, rank).
A uniform is the top 24 bits of a word times 2**-24, so it lies on a grid
that float32 and float64 both represent exactly.

Pins (tests/test_oracle_philox.py): bit-for-bit equality with numpy's own
``numpy.random.Philox`` (an independent Philox4x64-10) over many keys and
counters, with numpy's counter convention fixed by experiment; the uniform
grid and range.
"""

MASK64 = (1 << 64) - 1

# Multipliers and key increments of Philox4x64 (SC'11 paper, section 5).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1


def _mulhilo(a, b):
    prod = a * b
    return prod >> 64, prod & MASK64


def philox4x64_10(counter, key):
    """Philox4x64-10 bijection: 4x64-bit counter, 2x64-bit key -> 4 words."""
    c0, c1, c2, c3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for _ in range(10):
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & MASK64
        k1 = (k1 + PHILOX_W1) & MASK64
    return c0, c1, c2, c3


def uniform24(word):
    """Top 24 bits of a 64-bit word as a float in [0, 1 - 2**-24]."""
    return float(int(word) >> 40) * (2.0 ** -24)


def _uv(seed, tag, seq_id, pos, rank):
    w = philox4x64_10((seq_id, pos, rank, 0), (seed, tag))
    return uniform24(w[0]), uniform24(w[1])


def window_uniforms(seed, tag, seq_id, base_pos, gamma):
    """Uniforms of one window: u[i] decides draft i, v[i] samples the token
    produced at window position i (i = 0..gamma; u[gamma] is unused).

    Draft i sits at absolute position base_pos + 1 + i."""
    u, v = [], []
    for i in range(gamma + 1):
        a, b = _uv(seed, tag, seq_id, base_pos + 1 + i, 0)
        u.append(a)
        v.append(b)
    return u, v


def tree_uniforms(seed, tag, seq_id, base_pos, depth, rank):
    """Per-node uniforms of a token tree.

    u_node[v]: accept uniform of node v (v >= 1), keyed at its own
               position base_pos + depth(v) and its rank.
    v_node[v]: sampling uniform of the token emitted after node v, keyed at
               position base_pos + depth(v) + 1 and rank(v).
    A chain (branching 1) reproduces window_uniforms exactly."""
    n = len(depth)
    u_node = [0.0] * n
    v_node = [0.0] * n
    for v in range(n):
        if v > 0:
            u_node[v] = _uv(seed, tag, seq_id, base_pos + depth[v], rank[v])[0]
        v_node[v] = _uv(seed, tag, seq_id, base_pos + depth[v] + 1, rank[v])[1]
    return u_node, v_node
