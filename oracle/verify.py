"""Float64 definitions of speculative-decoding verification (test infrastructure).

One sequence at a time, numpy row operations, float64 throughout.  Nothing here
is blocked, fused or reordered beyond the definitions below.

Sources (page title, section):
* Speculative-sampling rule (accept when u < min(1, p/q), resample from the
  renormalised max(0, p - q) at the first rejection, bonus token from p after
  a full window): the rule the CLaSp review cites as lossless ("Assumptions &
  free parameters", last item) and the PipeSpec review cites through the
  Leviathan et al. expected-token formula ("Assumptions & free parameters").
* Greedy verification: the verifier makes its own single-token prediction and
  keeps the longest matching prefix (PipeSpec review, "What carries the
  argument"), at temperature 0 ("Reading between the lines").
* Rollback: on a mismatch, earlier stages roll their buffers back to the last
  verified token (PipeSpec review, "What carries the argument").
* Token tree and second speculative stage: "Accelerating LLM Inference with
  Staged Speculative Decoding", abstract.

Readings where the pages are silent:
* target logits carry gamma+1 rows (the last is the bonus row), draft logits
  gamma rows;
* the accept test is strict, written u*Q < P (equal to u < min(1, P/Q) since
  u < 1; Q = 0 accepts iff P > 0);
* the inverse CDF walks the vocabulary in index order and returns the smallest
  k with C_k > tau, tau = v * C_{V-1};
* greedy ties go to the smallest index; the greedy emitted token is the argmax
  of the first unmatched row;
* a tree node is accepted when its own test passes against its parent's row
  and its parent is accepted; the deepest accepted node wins, ties to the
  smallest node index;
* the lossless tree walk (verify_tree_multiround) tries siblings in index
  order, and after a rejection whose residual has no mass keeps the residual;
* rollback keeps a buffer that already agrees with the verified sequence and
  is at least as long, otherwise truncates it at the first divergence and
  appends the verified tail.

Pins: tests/test_oracle_*.py (brute-force exact laws at V=8, chi-square on
Philox-driven windows, the pages' expected-length and steady-state formulas on
exact-alpha inputs, scipy softmax/logsumexp, numpy argmax, special cases,
chain tree == window, brute-force tree paths, rollback invariants; for the
LM-head logits: one-hot unembeddings reduce it to the window on the hidden
values, and it is invariant under exact rescaling and vocabulary permutation;
multi-candidate walk: its exact output law equals the target's autoregressive
law on enumerated small trees, chain == window, and the closed form of the
residual after j rejections).
"""

import numpy as np

# --------------------------------------------------------------------------
# decoding and per-row probability
# --------------------------------------------------------------------------


def decode(raw, dtype):
    """Exact float64 values of a logits array.

    dtype 'bf16': raw holds the uint16 bit patterns (the high half of a
    float32); 'f16': uint16 bit patterns of IEEE half; 'f32' / 'f64': floats.
    """
    raw = np.asarray(raw)
    if dtype == "bf16":
        bits = raw.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return raw.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype in ("f32", "f64"):
        return raw.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def softmax(x):
    """Softmax of one row of float64 logits; -inf entries get probability 0."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    if not np.isfinite(m):
        raise ValueError("row has no finite logit")
    e = np.exp(x - m)
    return e / e.sum()


def first_argmax(x):
    """Index of the first maximal entry (-0 and +0 compare equal)."""
    x = np.asarray(x)
    return int(np.flatnonzero(x == x.max())[0])


# --------------------------------------------------------------------------
# inverse-CDF sampling
# --------------------------------------------------------------------------


def inverse_cdf(w, v):
    """Sample index of nonnegative weights w with uniform v in [0, 1).

    C_k is the running sum of w in index order; tau = v * C_{V-1}; the result
    is the smallest k with C_k > tau.  If rounding leaves no such k, the last
    index with w_k > 0 is returned.  Returns (k, info) where info holds tau,
    the total and the two CDF values around k (for margin reporting), or
    (None, None) when the total is 0.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    total = float(c[-1])
    if total <= 0.0:
        return None, None
    tau = v * total
    k = int(np.searchsorted(c, tau, side="right"))
    if k >= len(w):
        k = int(np.flatnonzero(w > 0)[-1])
    lo = float(c[k - 1]) if k > 0 else 0.0
    info = {"tau": tau, "Z": total, "C_lo": lo, "C_hi": float(c[k])}
    return k, info


# --------------------------------------------------------------------------
# stochastic window
# --------------------------------------------------------------------------


def verify_window(target, draft, tokens, length, u, v):
    """Speculative-sampling verification of one window.

    target: (gamma+1, V) float64 logits, row i = target's next-token logits
            after the context extended by drafts 0..i-1.
    draft:  (gamma, V) float64 logits the draft tokens were sampled from.
    tokens: gamma draft token ids.  length: drafts to verify, 0..gamma.
    u[i]:   accept uniform of draft i; v[i]: sampling uniform of the token
            produced at window position i.

    Returns a dict: n (accepted drafts), out (n accepted drafts then the
    corrected or bonus token), P[i] = p_i(x_i), Q[i] = q_i(x_i) for i < length,
    ratio[i] = P/Q of every examined position, u, and the sample record.
    """
    gamma = draft.shape[0]
    if not (0 <= length <= gamma):
        raise ValueError("length outside [0, gamma]")
    V = target.shape[1]
    P, Q = [], []
    for i in range(length):
        x = int(tokens[i])
        if not (0 <= x < V):
            raise ValueError("draft token outside the vocabulary")
        P.append(float(softmax(target[i])[x]))
        Q.append(float(softmax(draft[i])[x]))

    n = length
    ratios = []
    for i in range(length):
        ratios.append(P[i] / Q[i] if Q[i] > 0 else np.inf)
        if not (u[i] * Q[i] < P[i]):
            n = i
            break

    p_n = softmax(target[n])
    if n < length:
        w = np.maximum(0.0, p_n - softmax(draft[n]))
        kind = "residual"
        y, info = inverse_cdf(w, v[n])
        if y is None:  # no residual mass: unreachable after a real rejection
            kind = "residual-empty"
            y, info = inverse_cdf(p_n, v[n])
    else:
        kind = "bonus"
        y, info = inverse_cdf(p_n, v[n])
    out = [int(t) for t in tokens[:n]] + [int(y)]
    sample = dict(info)
    sample["kind"] = kind
    sample["y"] = int(y)
    return {
        "n": n,
        "out": out,
        "P": P,
        "Q": Q,
        "ratio": ratios,
        "u": list(u[:length]),
        "sample": sample,
    }


# --------------------------------------------------------------------------
# greedy window
# --------------------------------------------------------------------------


def verify_greedy(target, tokens, length):
    """Greedy (temperature-0) verification: keep the longest prefix of the
    drafts that equals the target's own argmax predictions, then emit the
    argmax of the first unmatched row (or of row `length` after a full match).
    """
    gamma = target.shape[0] - 1
    if not (0 <= length <= gamma):
        raise ValueError("length outside [0, gamma]")
    a = [first_argmax(target[i]) for i in range(length + 1)]
    n = length
    for i in range(length):
        if int(tokens[i]) != a[i]:
            n = i
            break
    return {"n": n, "out": [int(t) for t in tokens[:n]] + [a[n]], "argmax": a}


# --------------------------------------------------------------------------
# token tree
# --------------------------------------------------------------------------


def tree_meta(parent):
    """Depth, rank-within-depth and child flag of every node of a tree given
    by parent indices (parent[0] = -1, 0 <= parent[v] < v)."""
    N = len(parent)
    if N < 1 or parent[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    depth = [0] * N
    rank = [0] * N
    has_child = [False] * N
    count_at = {0: 1}
    for v in range(1, N):
        w = parent[v]
        if not (0 <= w < v):
            raise ValueError("parent index must precede its child")
        depth[v] = depth[w] + 1
        rank[v] = count_at.get(depth[v], 0)
        count_at[depth[v]] = rank[v] + 1
        has_child[w] = True
    return depth, rank, has_child


def verify_tree(target, draft, node_tokens, parent, mode, u_node, v_node):
    """Verification of a tree-shaped speculative batch.

    target[v]: target logits for the token after node v (row v).
    draft[v]:  draft logits the children of v were drawn from (stochastic).
    node_tokens[v]: token of node v (entry 0, the root, is ignored).
    mode: 'greedy' or 'stochastic'.  u_node / v_node as in tree_uniforms.

    Node v >= 1 is accepted when its parent w is accepted and its token passes
    the test against row w (argmax equality, or u_v * q_w < p_w); the deepest
    accepted node d (smallest index among equals) ends the path; the emitted
    token after d is argmax(target[d]) (greedy), a bonus draw from p_d when d
    has no children, or a draw from the renormalised max(0, p_d - q_d).
    Also returned: ok[v] (v and its ancestors accepted), own[v] (v's own
    test) and ratio[v] = P/Q of that test (stochastic mode), for reporting.
    """
    N = len(parent)
    depth, rank, has_child = tree_meta(parent)
    ok = [False] * N
    ok[0] = True
    own = [True] * N           # node v's own test against its parent's row
    ratio = [np.nan] * N       # P/Q of that test (stochastic mode)
    for v in range(1, N):
        w = parent[v]
        x = int(node_tokens[v])
        if not (0 <= x < target.shape[1]):
            raise ValueError("node token outside the vocabulary")
        if mode == "greedy":
            acc = x == first_argmax(target[w])
        else:
            P = float(softmax(target[w])[x])
            Q = float(softmax(draft[w])[x])
            ratio[v] = P / Q if Q > 0 else np.inf
            acc = u_node[v] * Q < P
        own[v] = bool(acc)
        ok[v] = ok[w] and acc
    d = 0
    for v in range(N):
        if ok[v] and depth[v] > depth[d]:
            d = v
    path = []
    w = d
    while w != 0:
        path.append(w)
        w = parent[w]
    path.reverse()
    sample = None
    if mode == "greedy":
        y = first_argmax(target[d])
    else:
        p_d = softmax(target[d])
        if has_child[d]:
            r = np.maximum(0.0, p_d - softmax(draft[d]))
            y, info = inverse_cdf(r, v_node[d])
            kind = "residual"
            if y is None:
                y, info = inverse_cdf(p_d, v_node[d])
                kind = "residual-empty"
        else:
            y, info = inverse_cdf(p_d, v_node[d])
            kind = "bonus"
        sample = dict(info)
        sample["kind"] = kind
        sample["y"] = int(y)
    return {
        "n": depth[d],
        "best": d,
        "path": path,
        "out": [int(node_tokens[v]) for v in path] + [int(y)],
        "ok": ok,
        "own": own,
        "ratio": ratio,
        "sample": sample,
    }


# --------------------------------------------------------------------------
# token tree, lossless multi-candidate walk
# --------------------------------------------------------------------------


def verify_tree_multiround(target, draft, node_tokens, parent, u_node, v_node):
    """Multi-candidate tree verification that keeps the target distribution.

    The pages cite this family only by title: SpecInfer, "tree-based
    speculative inference and verification" (PipeSpec review page, reference
    [16]; CLaSp review page, reference [29]).  This is that paper's published
    multi-round scheme, restated for one draft model whose sibling tokens are
    i.i.d. draws from the parent's draft row:

    Start at the root with r = p_w (w = current node).  Try the children of w
    in index order; child c with token x is accepted when u_c * q_w(x) < r(x)
    (u < min(1, r/q), strict as in the window).  On a rejection the residual
    becomes r <- max(0, r - q_w) / sum(max(0, r - q_w)); if that sum is 0 (only
    possible when r equals q_w) r is kept.  An accepted child becomes the new
    w and r restarts at its own p.  The walk ends at a leaf (bonus draw from
    p_w with v_w) or when every child of w was rejected (draw from r with v_w).

    Arguments as in verify_tree.  Returns n (depth of the final node), best
    (the final node), path, out (path tokens then the drawn token), tests (one
    record per sibling test: node, parent, u, ratio r(x)/q(x), r(x), q(x),
    the product `mass` of the normalisers applied to r so far and `shift`, the
    accumulated q-mass subtracted), and the sample record with the weights the
    final token was drawn from.
    """
    N = len(parent)
    depth, rank, has_child = tree_meta(parent)
    V = target.shape[1]
    for v in range(1, N):
        if not (0 <= int(node_tokens[v]) < V):
            raise ValueError("node token outside the vocabulary")
    children = [[] for _ in range(N)]
    for v in range(1, N):
        children[parent[v]].append(v)

    tests = []
    path = []
    w = 0
    while True:
        p_w = softmax(target[w])
        r = p_w
        mass, shift = 1.0, 0.0  # r == max(0, p_w - shift * q_w) / mass
        accepted = None
        if has_child[w]:
            q_w = softmax(draft[w])
            for c in children[w]:
                x = int(node_tokens[c])
                rx, qx = float(r[x]), float(q_w[x])
                tests.append({"node": c, "parent": w, "u": u_node[c],
                              "ratio": rx / qx if qx > 0 else np.inf,
                              "r": rx, "q": qx, "p": float(p_w[x]),
                              "mass": mass, "shift": shift})
                if u_node[c] * qx < rx:
                    accepted = c
                    break
                resid = np.maximum(0.0, r - q_w)
                z = float(resid.sum())
                if z > 0.0:
                    r = resid / z
                    shift += mass
                    mass *= z
        if accepted is None:
            break
        path.append(accepted)
        w = accepted

    y, info = inverse_cdf(r, v_node[w])
    if not has_child[w]:
        kind = "bonus"
    elif r is p_w:
        kind = "residual-empty"
    else:
        kind = "residual"
    sample = dict(info)
    sample["kind"] = kind
    sample["y"] = int(y)
    sample["weights"] = r
    sample["mass"] = mass
    sample["shift"] = shift
    return {
        "n": depth[w],
        "best": w,
        "path": path,
        "out": [int(node_tokens[v]) for v in path] + [int(y)],
        "tests": tests,
        "sample": sample,
    }


# --------------------------------------------------------------------------
# logits from hidden states (LM head) feeding the window
# --------------------------------------------------------------------------


def lmhead_logits(hidden, unembed):
    """Logits of each row of `hidden` (rows, H) against the unembedding
    `unembed` (V, H): logits[r, k] = sum_h hidden[r, h] * unembed[k, h], in
    float64 (products of bf16 values are exact in float64)."""
    hidden = np.asarray(hidden, dtype=np.float64)
    unembed = np.asarray(unembed, dtype=np.float64)
    return hidden @ unembed.T


def verify_window_lmhead(h_target, w_target, h_draft, w_draft, tokens, length, u, v):
    """The speculative-sampling window on logits produced from hidden states:
    target rows h_target (gamma+1, Ht) x w_target (V, Ht), draft rows
    h_draft (gamma, Hd) x w_draft (V, Hd); then verify_window."""
    return verify_window(lmhead_logits(h_target, w_target), lmhead_logits(h_draft, w_draft),
                         tokens, length, u, v)


# --------------------------------------------------------------------------
# rollback of per-stage buffers
# --------------------------------------------------------------------------


def rollback(buffers, lengths, stage, verified):
    """Roll the buffers of stages 0..stage-1 back to a verified sequence.

    buffers[j]: token list of stage j (only the first lengths[j] count).
    verified:   the verified token sequence of `stage` (length L).
    For each j < stage: m = first index < min(len_j, L) where the buffer
    disagrees with the verified sequence, else min(len_j, L).  If m < L the
    buffer becomes verified[0:L] (its tail after m is dropped) and len_j = L;
    otherwise it already holds verified[0:L] and is kept as it is.
    Returns new (buffers, lengths); buffers at or after `stage` are unchanged.
    """
    L = len(verified)
    new_bufs = [list(b) for b in buffers]
    new_lens = list(lengths)
    for j in range(stage):
        lj = lengths[j]
        lim = min(lj, L)
        m = lim
        for t in range(lim):
            if buffers[j][t] != verified[t]:
                m = t
                break
        if m < L:
            buf = new_bufs[j]
            if len(buf) < L:
                buf.extend([0] * (L - len(buf)))
            for t in range(m, L):
                buf[t] = int(verified[t])
            new_lens[j] = L
    return new_bufs, new_lens


# --------------------------------------------------------------------------
# three-stage hierarchy (PipeSpec-shaped, one stream)
# --------------------------------------------------------------------------


def hierarchy_three_stage(F, S1, S0, o0, gamma1, gamma2, mode, uv1, uv2, cap=16):
    """One stream of a k=3 hierarchy M0 -> M1 -> M2 (PipeSpec review, "What
    carries the argument"; second stage of speculation per the Staged
    Speculative Decoding abstract).

    F:  (gamma1+1, V) final-model logits, S1: (gamma1+1, V) stage-1 logits,
    S0: (gamma1, V) stage-0 logits; o0: gamma1 stage-0 draft tokens.
    Stage 1 verifies o0 against S1 with S0 as the draft distribution; stage 0's
    buffer is rolled back to stage 1's output O1.  Stage 2 verifies the first
    min(gamma2, len(O1)) tokens of O1 against F with S1 as the draft
    distribution; stages 0 and 1 are rolled back to its output O2.
    uv1 / uv2: (u, v) uniform lists of stage 1 / stage 2 windows.
    Buffers have `cap` slots; slots past a buffer's length start at 0.
    Returns O1, O2 and the rolled-back buffers.
    """
    def slots(seq):
        return list(seq) + [0] * (cap - len(seq))

    if mode == "greedy":
        r1 = verify_greedy(S1, o0, gamma1)
    else:
        r1 = verify_window(S1, S0, o0, gamma1, uv1[0], uv1[1])
    O1 = r1["out"]
    bufs = [slots(o0), slots(O1), slots([])]
    lens = [len(o0), len(O1), 0]
    bufs, lens = rollback(bufs, lens, 1, O1)
    len2 = min(gamma2, len(O1))
    toks2 = list(O1[:len2]) + [0] * (gamma2 - len2)
    if mode == "greedy":
        r2 = verify_greedy(F[: gamma2 + 1], toks2, len2)
    else:
        r2 = verify_window(F[: gamma2 + 1], S1[:gamma2], toks2, len2, uv2[0], uv2[1])
    O2 = r2["out"]
    bufs[2] = slots(O2)
    lens[2] = len(O2)
    bufs, lens = rollback(bufs, lens, 2, O2)
    return {"stage1": r1, "stage2": r2, "O1": O1, "O2": O2, "buffers": bufs, "lengths": lens}
