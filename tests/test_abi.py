"""The C-ABI library loads, exports every function include/sv.h declares, and
rejects bad host arguments before touching a device (no compute calls here)."""
import ctypes
import os
import re

import pytest

from draft_token_verification_06_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "sv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported_and_bound():
    L = _lib.lib()
    names = _declared()
    assert "sv_verify_window" in names and "sv_rollback" in names
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(_lib.EXPORTED)


def test_single_hip_runtime_is_mapped():
    _lib.lib()
    assert len(_lib.hip_runtime_paths()) == 1


def test_version_and_error_strings():
    L = _lib.lib()
    assert L.sv_version() == 10100
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert L.sv_strerror(st)
    assert L.sv_strerror(-99) == b"unknown status"


def test_workspace_size_rules():
    L = _lib.lib()
    assert L.sv_workspace_size(0, 256, 8, 128256, 1) > 0
    assert L.sv_workspace_size(0, 256, 8, 128256, 1) % 256 == 0
    assert L.sv_workspace_size(0, 0, 8, 100, 1) == 0
    assert L.sv_workspace_size(0, 1, 65, 100, 1) == 0
    assert L.sv_workspace_size(1, 1, 4, 100, 7) == 0
    assert L.sv_workspace_size(2, 1, 257, 100, 1) == 0
    assert L.sv_workspace_size(9, 1, 4, 100, 1) == 0


def test_tree_depth_and_malformed_parents():
    L = _lib.lib()
    arr = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    assert L.sv_tree_max_depth(arr([-1, 0, 0, 1, 3]), 5) == 3
    assert L.sv_tree_max_depth(arr([-1]), 1) == 0
    assert L.sv_tree_max_depth(arr([0, 0]), 2) == -4
    assert L.sv_tree_max_depth(arr([-1, 1]), 2) == -4
    assert L.sv_tree_max_depth(arr([-1] + list(range(64))), 65) == 64
    assert L.sv_tree_max_depth(arr([-1] + list(range(65))), 66) == -4
    assert L.sv_tree_max_depth(arr([-1] + [0] * 256), 257) == -4


def test_bad_host_arguments_return_status_without_device_work():
    L = _lib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # unknown dtype
    assert L.sv_verify_window(fake, 0, fake, 0, 5, fake, None, 1, 4, 100, 0, 0, None, None,
                              fake, fake, None, None, fake, 1 << 20, None) == -2
    # gamma out of range, null tokens, B = 0
    assert L.sv_verify_window(fake, 0, fake, 0, 1, fake, None, 1, 65, 100, 0, 0, None, None,
                              fake, fake, None, None, fake, 1 << 20, None) == -1
    assert L.sv_verify_window(fake, 0, fake, 0, 1, None, None, 1, 4, 100, 0, 0, None, None,
                              fake, fake, None, None, fake, 1 << 20, None) == -1
    assert L.sv_verify_greedy(fake, 0, 1, fake, None, 0, 4, 100, fake, fake, fake, 1 << 20,
                              None) == -1
    # misaligned bf16 logits
    odd = ctypes.c_void_p(0x1001)
    assert L.sv_verify_greedy(odd, 0, 1, fake, None, 1, 4, 100, fake, fake, fake, 1 << 20,
                              None) == -1
    # stride smaller than the rows it must hold
    assert L.sv_verify_greedy(fake, 10, 1, fake, None, 1, 4, 100, fake, fake, fake, 1 << 20,
                              None) == -1
    # workspace: missing, misaligned, too small
    assert L.sv_verify_greedy(fake, 0, 1, fake, None, 1, 4, 100, fake, fake, None, 1 << 20,
                              None) == -3
    assert L.sv_verify_greedy(fake, 0, 1, fake, None, 1, 4, 100, fake, fake,
                              ctypes.c_void_p(0x1010), 1 << 20, None) == -3
    assert L.sv_verify_greedy(fake, 0, 1, fake, None, 1, 4, 100, fake, fake, fake, 16,
                              None) == -3
    # tree: malformed parents, bad mode, stochastic without draft
    par = (ctypes.c_int32 * 3)(-1, 0, 5)
    assert L.sv_verify_tree(fake, fake, 1, fake, par, 1, 3, 100, 1, 0, 0, None, None,
                            fake, fake, fake, fake, fake, 1 << 20, None) == -4
    par = (ctypes.c_int32 * 3)(-1, 0, 1)
    assert L.sv_verify_tree(fake, fake, 1, fake, par, 1, 3, 100, 7, 0, 0, None, None,
                            fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert L.sv_verify_tree(fake, None, 1, fake, par, 1, 3, 100, 1, 0, 0, None, None,
                            fake, fake, fake, fake, fake, 1 << 20, None) == -1
    # multi-candidate walk without draft logits
    assert L.sv_verify_tree(fake, None, 1, fake, par, 1, 3, 100, 2, 0, 0, None, None,
                            fake, fake, fake, fake, fake, 1 << 20, None) == -1
    assert L.sv_verify_tree(fake, fake, 1, fake, par, 1, 3, 100, 3, 0, 0, None, None,
                            fake, fake, fake, fake, fake, 1 << 20, None) == -1
    # LM-head window: hidden width not a multiple of 64, null unembedding, small workspace
    assert L.sv_verify_window_lmhead(fake, fake, 100, fake, fake, 64, fake, None, 1, 4, 100,
                                     0, 0, None, None, fake, fake, None, None,
                                     fake, 1 << 30, None) == -1
    assert L.sv_verify_window_lmhead(fake, None, 64, fake, fake, 64, fake, None, 1, 4, 100,
                                     0, 0, None, None, fake, fake, None, None,
                                     fake, 1 << 30, None) == -1
    assert L.sv_verify_window_lmhead(fake, fake, 64, fake, fake, 64, fake, None, 1, 4, 100,
                                     0, 0, None, None, fake, fake, None, None,
                                     fake, 16, None) == -3
    assert L.sv_workspace_size(3, 4, 8, 1000, 0) == 0  # LM-head workspace is for bf16 only
    assert L.sv_workspace_size(3, 4, 8, 1000, 1) > 2 * 4 * 1000 * 4
    # rollback: stage outside [1, K-1], null buffers
    assert L.sv_rollback(fake, fake, 4, 3, 8, 3, fake, 8, fake, 0, None) == -1
    assert L.sv_rollback(fake, fake, 4, 3, 8, 0, fake, 8, fake, 0, None) == -1
    assert L.sv_rollback(None, fake, 4, 3, 8, 1, fake, 8, fake, 0, None) == -1
    assert L.sv_probe_read(fake, 17, fake, None) == -1
    # no-allocation window: host checks, and a call beyond the static scratch
    assert L.sv_verify_window_noalloc(fake, 0, fake, 0, 5, fake, None, 1, 4, 100, 0, 0, None, None,
                                      fake, fake, None, None, None) == -2
    assert L.sv_verify_window_noalloc(fake, 0, fake, 0, 1, fake, None, 1, 65, 100, 0, 0, None, None,
                                      fake, fake, None, None, None) == -1
    need = L.sv_workspace_size(0, 4096, 64, 1 << 21, 1)
    assert need > 8 << 20
    assert L.sv_verify_window_noalloc(fake, 0, fake, 0, 1, fake, None, 4096, 64, 1 << 21, 0, 0, None, None,
                                      fake, fake, None, None, None) == -6


def test_grids_beyond_a_dispatch_are_rejected_on_the_host():
    """A dispatch counts each grid dimension in 32-bit work-items.  Calls whose
    row pass (256 work-items per row segment) or draw (1024 per sequence)
    would not fit return SV_EINVAL before the workspace is examined; one
    sequence fewer passes that check and meets the (deliberately too small)
    workspace instead, SV_EWORKSPACE.  Nothing is launched either way."""
    L = _lib.lib()
    fake = ctypes.c_void_p(0x1000)

    def window(B):
        return L.sv_verify_window(fake, 0, fake, 0, 1, fake, None, B, 1, 8, 0, 0, None, None,
                                  fake, fake, None, None, fake, 1 << 20, None)

    # draw: 2^22 sequences x 1024 work-items = 2^32 (the row pass, 3 x 2^22 segments, fits)
    assert window(1 << 22) == -1
    assert window((1 << 22) - 1) == -3
    assert L.sv_verify_window_early_exit(fake, 0, fake, 0, 1, fake, None, 1 << 22, 1, 8, 0, 0, None, None,
                                         fake, fake, None, None, fake, 1 << 20, None) == -1

    # row pass: B x 9 rows (gamma = 8, one segment at V = 8) x 256 work-items
    def greedy(B):
        return L.sv_verify_greedy(fake, 0, 1, fake, None, B, 8, 8, fake, fake, fake, 1 << 20, None)

    limit = ((1 << 24) - 1) // 9
    assert greedy(limit) == -3
    assert greedy(limit + 1) == -1

    # tree: 2N rows per sequence in the layout, 1024 work-items per sequence when sampling
    par = (ctypes.c_int32 * 2)(-1, 0)
    assert L.sv_verify_tree(fake, fake, 1, fake, par, 1 << 22, 2, 8, 1, 0, 0, None, None,
                            fake, fake, fake, fake, fake, 1 << 20, None) == -1

    # LM-head window: the draw's grid at 2^22 sequences
    def lmhead(B):
        return L.sv_verify_window_lmhead(fake, fake, 64, fake, fake, 64, fake, None, B, 1, 256,
                                         0, 0, None, None, fake, fake, None, None, fake, 1 << 30, None)

    assert lmhead(1 << 22) == -1
    assert lmhead((1 << 22) - 1) == -3

    # rollback: one wavefront per stream, 2^26 streams = 2^32 work-items
    assert L.sv_rollback(fake, fake, 1 << 26, 3, 8, 1, fake, 8, fake, 0, None) == -1


def test_binding_rejects_host_tensors_before_any_call():
    """The Python binding checks tensors on the host: logits, tokens and
    outputs in host memory are refused with ValueError, before the library is
    asked to do anything."""
    import torch
    import draft_token_verification_06_amd as sv

    B, gamma, V = 2, 3, 16
    t = torch.zeros(B, gamma + 1, V, dtype=torch.bfloat16)
    d = torch.zeros(B, gamma, V, dtype=torch.bfloat16)
    toks = torch.zeros(B, gamma, dtype=torch.int32)
    with pytest.raises(ValueError):
        sv.verify_window(t, d, toks)
    with pytest.raises(ValueError):
        sv.verify_greedy(t, toks)
    with pytest.raises(ValueError):
        sv.verify_window(t.to(torch.float64), d, toks)
    with pytest.raises(ValueError):
        sv.verify_window(t[:, :gamma], d, toks)          # target needs gamma + 1 rows
    with pytest.raises(ValueError):
        sv.rollback(torch.zeros(2, 3, 4, dtype=torch.int32), torch.zeros(2, 3, dtype=torch.int32), 1,
                    torch.zeros(2, 4, dtype=torch.int32), torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        sv.probe_read(torch.zeros(1024, dtype=torch.uint8))
