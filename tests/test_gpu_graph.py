"""The entry points under HIP graph capture: a window, a greedy window and an
early-exit window captured once and replayed several times, with eager work and
synchronisations between replays; every replay equals the eager result bit
for bit.  The library records no memset, allocation or synchronisation, so
its launches are capturable as they are."""
import pytest
import torch

import draft_token_verification_06_amd as sv
from draft_token_verification_06_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replays_match(make_call, outputs, reps=4):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        make_call()  # eager on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        make_call()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outputs:
            o.fill_(-7)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w), r


def test_window_graph_replays():
    print("graph window", flush=True)
    d = synth.window_batch(8, 8, 128256, "bf16", 3.0, 6.0, 1.0, seed=1002, device=DEV)
    ws = sv.workspace(sv.SV_OP_WINDOW, 8, 8, 128256, torch.bfloat16, DEV)
    out = sv.WindowResult(torch.empty(8, dtype=torch.int32, device=DEV),
                          torch.empty(8, 9, dtype=torch.int32, device=DEV),
                          torch.empty(8, 8, dtype=torch.float32, device=DEV),
                          torch.empty(8, 8, dtype=torch.float32, device=DEV))
    _replays_match(lambda: sv.verify_window(d["target"], d["draft"], d["tokens"], seed=3, ws=ws, out=out),
                   [out.n_accepted, out.out_tokens, out.p_draft, out.q_draft])


def test_greedy_and_early_exit_graph_replays():
    print("graph greedy/early exit", flush=True)
    d = synth.window_batch(16, 8, 32000, "bf16", 3.0, 6.0, 0.5, seed=5, device=DEV)
    wsg = sv.workspace(sv.SV_OP_GREEDY, 16, 8, 32000, torch.bfloat16, DEV)
    outg = sv.WindowResult(torch.empty(16, dtype=torch.int32, device=DEV),
                           torch.empty(16, 9, dtype=torch.int32, device=DEV))
    _replays_match(lambda: sv.verify_greedy(d["target"], d["tokens"], ws=wsg, out=outg),
                   [outg.n_accepted, outg.out_tokens])
    ws = sv.workspace(sv.SV_OP_WINDOW, 16, 8, 32000, torch.bfloat16, DEV)
    out = sv.WindowResult(torch.empty(16, dtype=torch.int32, device=DEV),
                          torch.empty(16, 9, dtype=torch.int32, device=DEV))
    _replays_match(lambda: sv.verify_window(d["target"], d["draft"], d["tokens"], seed=1, ws=ws, out=out,
                                            early_exit=True),
                   [out.n_accepted, out.out_tokens])


def test_noalloc_window_graph_replays():
    """The no-allocation window (its workspace is the library's static device
    array) captured and replayed: every replay equals the eager result."""
    print("graph no-alloc window", flush=True)
    d = synth.window_batch(8, 8, 128256, "bf16", 3.0, 6.0, 1.0, seed=1003, device=DEV)
    out = sv.WindowResult(torch.empty(8, dtype=torch.int32, device=DEV),
                          torch.empty(8, 9, dtype=torch.int32, device=DEV),
                          torch.empty(8, 8, dtype=torch.float32, device=DEV),
                          torch.empty(8, 8, dtype=torch.float32, device=DEV))
    _replays_match(lambda: sv.verify_window_noalloc(d["target"], d["draft"], d["tokens"], seed=4, out=out),
                   [out.n_accepted, out.out_tokens, out.p_draft, out.q_draft])
