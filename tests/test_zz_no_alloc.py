"""sv_verify_window_noalloc (the window on the library's static per-GPU
scratch, for callers that cannot allocate) against sv_verify_window with a
caller workspace: bit-identical outputs on two calls in a row, the second
with a smaller input, and the second also against the float64 oracle."""
import numpy as np
import pytest
import torch

import draft_token_verification_06_amd as sv
from draft_token_verification_06_amd import synth
from gpu_common import check_window, max_margins

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b):
    for x, y in ((a.n_accepted, b.n_accepted), (a.out_tokens, b.out_tokens),
                 (a.p_draft, b.p_draft), (a.q_draft, b.q_draft)):
        assert torch.equal(x, y)


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    print("no-alloc: B=256 gamma=8 V=128256 bf16, then B=8 gamma=4 V=32000 f32", flush=True)
    d1 = synth.window_config5(0.6, device=DEV)
    kw1 = dict(seed=3, tag=1, return_probs=True)
    want1 = sv.verify_window(d1["target"], d1["draft"], d1["tokens"], **kw1)
    got1 = sv.verify_window_noalloc(d1["target"], d1["draft"], d1["tokens"], **kw1)
    torch.cuda.synchronize()
    _same(want1, got1)

    rng = np.random.default_rng(5)
    d2 = synth.window_batch(8, 4, 32000, "f32", target_sd=2.0, boost=0.0, sigma=0.5, seed=12,
                            device=DEV)
    wl = torch.tensor([4, 0, 3, 4, 1, 2, 4, 4], dtype=torch.int32, device=DEV)
    sid = torch.from_numpy(rng.integers(0, 2 ** 40, 8).astype(np.int64)).to(DEV)
    bp = torch.from_numpy(rng.integers(0, 10 ** 6, 8).astype(np.int64)).to(DEV)
    kw2 = dict(seed=11, tag=2, window_len=wl, seq_ids=sid, base_pos=bp, return_probs=True)
    got2 = sv.verify_window_noalloc(d2["target"], d2["draft"], d2["tokens"], **kw2)
    want2 = sv.verify_window(d2["target"], d2["draft"], d2["tokens"], **kw2)
    torch.cuda.synchronize()
    _same(want2, got2)
    n, m = check_window(d2, got2, seed=11, tag=2, window_len=wl, seq_ids=sid, base_pos=bp)
    assert m <= max_margins(8)
    # the first input again after the smaller one: nothing carries over
    again = sv.verify_window_noalloc(d1["target"], d1["draft"], d1["tokens"], **kw1)
    torch.cuda.synchronize()
    _same(want1, again)
