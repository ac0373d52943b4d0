"""GPU parity of sv_verify_tree (bit-exact greedy, stochastic within the margin
rule) and sv_rollback (bit-exact), including the PipeSpec-shaped hierarchy."""
import numpy as np
import pytest
import torch

import oracle
import draft_token_verification_06_amd as sv
from draft_token_verification_06_amd import synth
from gpu_common import (check_tree, check_window, check_greedy, host_rows, max_margins,
                        window_case_in_margin, window_divergence)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_tree_branching_4_3_2_v50257_f16(mode):
    print("tree", mode, flush=True)
    d = synth.tree_config3(device=DEV)
    res = sv.verify_tree(d["target"], d["draft"], d["tokens"], d["parent"], mode=mode, seed=0)
    n, m = check_tree(d, res, mode, seed=0)
    assert m == 0 or mode == "stochastic"


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_tree_branching_4_3_2_at_b256_every_sequence(mode):
    # 256 sequences: the stochastic draw runs one workgroup per sequence, each
    # deciding its own tree; the greedy tree runs the standalone decision
    print("tree B=256", mode, flush=True)
    d = synth.tree_batch(256, synth.bfs_tree((4, 3, 2)), 50257, dtype="f16", sigma=0.5, seed=4256,
                         device=DEV)
    res = sv.verify_tree(d["target"], d["draft"], d["tokens"], d["parent"], mode=mode, seed=11)
    n, m = check_tree(d, res, mode, seed=11)
    print("tree B=256", mode, "margin cases", m, "of", n, flush=True)
    assert m == 0 or (mode == "stochastic" and m <= max_margins(256))


@pytest.mark.parametrize("B", [4, 256])
@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_tree_caller_keys(mode, B):
    """Per-node trees keyed by the caller: random seq_ids, base_pos and a tag
    other than 0.  B = 4 takes the split draw (several workgroups per
    sequence, each deciding its tree), B = 256 one workgroup per sequence.  A
    run with other keys must change the stochastic outcome somewhere."""
    print("tree caller keys", mode, B, flush=True)
    rng = np.random.default_rng(17 + B)
    d = synth.tree_batch(B, synth.bfs_tree((4, 3, 2)), 50257, dtype="f16", sigma=0.5, seed=5000 + B,
                         device=DEV)
    sid = torch.from_numpy(rng.integers(0, 2 ** 62, B).astype(np.int64)).to(DEV)
    bp = torch.from_numpy(rng.integers(0, 10 ** 9, B).astype(np.int64)).to(DEV)
    seed, tag = int(rng.integers(0, 2 ** 63)), int(rng.integers(1, 2 ** 63))
    res = sv.verify_tree(d["target"], d["draft"], d["tokens"], d["parent"], mode=mode, seed=seed,
                         tag=tag, seq_ids=sid, base_pos=bp)
    n, m = check_tree(d, res, mode, seed=seed, tag=tag, seq_ids=sid, base_pos=bp)
    print("tree caller keys", mode, B, "margin cases", m, "of", n, flush=True)
    assert m == 0 or (mode == "stochastic" and m <= max_margins(B))
    if mode == "stochastic" and B == 256:
        other = sv.verify_tree(d["target"], d["draft"], d["tokens"], d["parent"], mode=mode, seed=seed,
                               tag=tag, seq_ids=sid + 1, base_pos=bp)
        assert not torch.equal(other.out_tokens, res.out_tokens)


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_tree_greedy_friendly_tokens_reach_deep_nodes(mode):
    # half of the node tokens equal the parent's argmax, so long paths occur
    d = synth.tree_batch(16, synth.bfs_tree((3, 2, 2, 1)), 3001, dtype="bf16", sigma=0.3,
                         seed=21, device=DEV)
    am = d["target"].float().argmax(-1).to(torch.int32)
    par = torch.tensor([max(p, 0) for p in d["parent"]], device=DEV)
    take = torch.rand(d["tokens"].shape, device=DEV) < 0.6
    toks = torch.where(take, am[:, par], d["tokens"])
    toks[:, 0] = 0
    d["tokens"] = toks.contiguous()
    res = sv.verify_tree(d["target"], d["draft"], d["tokens"], d["parent"], mode=mode, seed=4)
    check_tree(d, res, mode, seed=4)
    if mode == "greedy":
        assert res.n_accepted.max().item() >= 2


def test_chain_tree_equals_window():
    B, gamma, V = 12, 6, 5000
    d = synth.window_batch(B, gamma, V, "bf16", sigma=0.4, seed=31, device=DEV)
    parent = [-1] + list(range(gamma))
    t = d["target"]
    dr = torch.cat([d["draft"], d["draft"][:, :1]], dim=1).contiguous()  # leaf row unused
    nt = torch.cat([torch.zeros(B, 1, dtype=torch.int32, device=DEV), d["tokens"]], 1).contiguous()
    w = sv.verify_window(t, d["draft"], d["tokens"], seed=7)
    tr = sv.verify_tree(t, dr, nt, parent, mode="stochastic", seed=7)
    assert torch.equal(w.n_accepted, tr.n_accepted)
    assert torch.equal(w.out_tokens, tr.out_tokens)
    wg = sv.verify_greedy(t, d["tokens"])
    tg = sv.verify_tree(t, None, nt, parent, mode="greedy")
    assert torch.equal(wg.out_tokens, tg.out_tokens)


def test_tree_invalid_node_token_and_bad_parent():
    d = synth.tree_batch(3, synth.bfs_tree((2, 2)), 100, dtype="f32", seed=2, device=DEV)
    toks = d["tokens"].clone()
    toks[1, 4] = 100
    res = sv.verify_tree(d["target"], d["draft"], toks, d["parent"], mode="stochastic")
    assert res.n_accepted[1].item() == -1 and torch.all(res.out_tokens[1] == -1)
    assert res.n_accepted[0].item() >= 0
    with pytest.raises(sv.SvError) as e:
        sv.verify_tree(d["target"], d["draft"], toks, [-1, 0, 2, 1, 1, 2, 2], mode="greedy")
    assert e.value.status == -4
    # the same with a vocabulary that splits the draw over several workgroups
    # per sequence (every one of them decides; the first writes the outputs)
    d = synth.tree_batch(3, synth.bfs_tree((2, 2)), 20000, dtype="f16", seed=5, device=DEV)
    toks = d["tokens"].clone()
    toks[2, 3] = -7
    res = sv.verify_tree(d["target"], d["draft"], toks, d["parent"], mode="stochastic", seed=4)
    assert res.n_accepted[2].item() == -1 and torch.all(res.out_tokens[2] == -1)
    assert res.best_node[2].item() == -1
    dd = dict(d, tokens=toks)
    check_tree(dd, res, "stochastic", seed=4, rows=[0, 1])


def _rollback_case(rng, S, K, cap):
    bufs = rng.integers(0, 5, (S, K, cap)).astype(np.int32)
    lens = rng.integers(0, cap + 1, (S, K)).astype(np.int32)
    L = rng.integers(0, cap + 1, S).astype(np.int32)
    ver = rng.integers(0, 5, (S, cap + 3)).astype(np.int32)
    for s in range(S):  # frequent agreement with the verified prefix
        for j in range(K):
            a = int(rng.integers(0, min(lens[s, j], L[s]) + 1))
            if rng.uniform() < 0.6:
                bufs[s, j, :a] = ver[s, :a]
    return bufs, lens, ver, L


@pytest.mark.parametrize("cap", [1, 9, 64, 200])
def test_rollback_bit_exact(cap):
    rng = np.random.default_rng(cap)
    S, K = 257, 4
    bufs, lens, ver, L = _rollback_case(rng, S, K, cap)
    lens[3, 0] = cap + 1  # invalid length -> -1, tokens untouched
    for stage in (1, 2, 3):
        bt = torch.tensor(bufs, device=DEV)
        bl = torch.tensor(lens, device=DEV)
        sv.rollback(bt, bl, stage, torch.tensor(ver, device=DEV), torch.tensor(L - 1, device=DEV),
                    len_offset=1)
        gb, gl = bt.cpu().numpy(), bl.cpu().numpy()
        for s in range(S):
            if s == 3 and stage >= 1:
                assert gl[3, 0] == -1 and np.array_equal(gb[3, 0], bufs[3, 0])
                nb, nl = oracle.rollback([list(x) for x in bufs[s, 1:]], list(lens[s, 1:]),
                                         stage - 1, list(ver[s, :L[s]]))
                assert [list(x) for x in gb[s, 1:]] == nb and list(gl[s, 1:]) == nl
                continue
            nb, nl = oracle.rollback([list(x) for x in bufs[s]], list(lens[s]), stage,
                                     list(ver[s, :L[s]]))
            assert [list(x) for x in gb[s]] == nb, (s, stage)
            assert list(gl[s]) == nl, (s, stage)


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
def test_three_stage_hierarchy_small_vocab(mode):
    # 64 streams of the PipeSpec-shaped hierarchy at V = 2048 (full size runs in
    # the full-size tests): verify stage 1, roll back, verify stage 2, roll back.
    S, V, g1, g2, cap = 64, 2048, 8, 4, 16
    h = synth.hierarchy_config4(S=S, V=V, mode=mode, seed=5, device=DEV)
    m = run_hierarchy_and_check(h, g1, g2, cap, mode, rows=range(S))
    assert m <= 1


def run_hierarchy_and_check(h, g1, g2, cap, mode, rows):
    S = h["S"]
    F, S1, S0, o0 = h["F"], h["S1"], h["S0"], h["o0"]
    bt = torch.zeros(S, 3, cap, dtype=torch.int32, device=DEV)
    bl = torch.zeros(S, 3, dtype=torch.int32, device=DEV)
    bt[:, 0, :g1] = o0
    bl[:, 0] = g1
    if mode == "greedy":
        r1 = sv.verify_greedy(S1, o0)
    else:
        r1 = sv.verify_window(S1, S0, o0, seed=0, tag=1)
    bt[:, 1, : g1 + 1] = r1.out_tokens.clamp(min=0)  # slots past the length hold 0
    bl[:, 1] = r1.n_accepted + 1
    sv.rollback(bt, bl, 1, r1.out_tokens, r1.n_accepted, len_offset=1)
    wl2 = torch.clamp(r1.n_accepted + 1, max=g2).to(torch.int32)
    toks2 = r1.out_tokens[:, :g2].contiguous()
    if mode == "greedy":
        r2 = sv.verify_greedy(F[:, : g2 + 1], toks2, window_len=wl2)
    else:
        r2 = sv.verify_window(F[:, : g2 + 1], S1[:, :g2], toks2, seed=0, tag=2, window_len=wl2)
    bt[:, 2, : g2 + 1] = r2.out_tokens.clamp(min=0)
    bl[:, 2] = r2.n_accepted + 1
    sv.rollback(bt, bl, 2, r2.out_tokens, r2.n_accepted, len_offset=1)
    torch.cuda.synchronize()
    gb, gl = bt.cpu().numpy(), bl.cpu().numpy()
    o0h = o0.cpu().numpy()
    n1, out1 = r1.n_accepted.cpu().numpy(), r1.out_tokens.cpu().numpy()
    n2, out2 = r2.n_accepted.cpu().numpy(), r2.out_tokens.cpu().numpy()
    toks2h = toks2.cpu().numpy()
    margins = 0
    for s in rows:
        Fh = host_rows(F[s], h["dtype"])
        S1h = host_rows(S1[s], h["dtype"])
        S0h = host_rows(S0[s], h["dtype"])
        uv1 = oracle.window_uniforms(0, 1, s, 0, g1)
        uv2 = oracle.window_uniforms(0, 2, s, 0, g2)
        o = oracle.hierarchy_three_stage(Fh, S1h, S0h, list(o0h[s]), g1, g2, mode, uv1, uv2, cap)
        # stage 1 must match unless a margin case at the point of divergence
        # explains it; then stop for this stream
        div = window_divergence(o["stage1"], int(n1[s]), out1[s], g1, o0h[s], Fh.shape[1])
        if div is not None:
            assert mode == "stochastic" and window_case_in_margin(o["stage1"], div), (s, "stage 1", div)
            margins += 1
            continue
        div = window_divergence(o["stage2"], int(n2[s]), out2[s], g2, toks2h[s], Fh.shape[1])
        if div is not None:
            assert mode == "stochastic" and window_case_in_margin(o["stage2"], div), (s, "stage 2", div)
            margins += 1
            continue
        assert [list(x) for x in gb[s]] == o["buffers"], s
        assert list(gl[s]) == o["lengths"], s
    return margins
