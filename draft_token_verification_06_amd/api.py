"""Python binding of the C ABI in include/sv.h: argument marshalling only.

Tensors must live on a ROCm device; every computation runs in the HIP
library on the current torch stream of that device.  Results come back as
device tensors; nothing synchronises.
"""
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import lib

SV_OP_WINDOW, SV_OP_GREEDY, SV_OP_TREE, SV_OP_LMHEAD = 0, 1, 2, 3
SV_TREE_GREEDY, SV_TREE_STOCHASTIC, SV_TREE_MULTI_CANDIDATE = 0, 1, 2
_TREE_MODES = {"greedy": SV_TREE_GREEDY, "stochastic": SV_TREE_STOCHASTIC,
               "multi_candidate": SV_TREE_MULTI_CANDIDATE}
_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class SvError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"specverify status {status}: {lib().sv_strerror(status).decode()}")


def _check(status):
    if status != 0:
        raise SvError(status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _logits(t, rows, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in _DTYPE_CODE:
        raise ValueError(f"{name}: dtype {t.dtype} is not float32, bfloat16 or float16")
    if t.dim() != 3 or t.shape[1] != rows:
        raise ValueError(f"{name}: expected shape (B, {rows}, V), got {tuple(t.shape)}")
    V = t.shape[2]
    if t.stride(2) != 1 or t.stride(1) != V:
        raise ValueError(f"{name}: rows of one sequence must be contiguous")
    return t.stride(0)


def _i32(t, shape, name):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous int32 device tensor of shape {tuple(shape)}")


def _optional(t, dtype, B, name):
    if t is None:
        return None
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (B,):
        raise ValueError(f"{name}: expected a contiguous {dtype} device tensor of shape ({B},)")
    return t


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _ws_bytes(ws, dev):
    """Byte size of a caller-supplied workspace (a contiguous device tensor)."""
    if not ws.is_cuda or not ws.is_contiguous() or ws.device != dev:
        raise ValueError(f"workspace: expected a contiguous device tensor on {dev}")
    return ws.numel() * ws.element_size()


def _out_tensor(t, dtype, shape, dev, name):
    if t is None:
        return
    if t.dtype != dtype or t.device != dev or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)} on {dev}")


def _check_window_out(out, B, gamma, dev):
    if out.n_accepted is None or out.out_tokens is None:
        raise ValueError("n_accepted and out_tokens are required outputs")
    _out_tensor(out.n_accepted, torch.int32, (B,), dev, "n_accepted")
    _out_tensor(out.out_tokens, torch.int32, (B, gamma + 1), dev, "out_tokens")
    _out_tensor(out.p_draft, torch.float32, (B, gamma), dev, "p_draft")
    _out_tensor(out.q_draft, torch.float32, (B, gamma), dev, "q_draft")


def workspace_size(op, B, n, V, dtype):
    return int(lib().sv_workspace_size(op, B, n, V, _DTYPE_CODE[dtype]))


def workspace(op, B, n, V, dtype, device):
    nbytes = workspace_size(op, B, n, V, dtype)
    if nbytes == 0:
        raise ValueError("invalid sizes for a workspace")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class WindowResult:
    n_accepted: torch.Tensor
    out_tokens: torch.Tensor
    p_draft: Optional[torch.Tensor] = None
    q_draft: Optional[torch.Tensor] = None


@dataclass
class TreeResult:
    n_accepted: torch.Tensor
    best_node: torch.Tensor
    out_tokens: torch.Tensor
    out_nodes: torch.Tensor


SV_PART_ROW_STATS, SV_PART_DECIDE_SAMPLE = 1, 2


def verify_window(target, draft, tokens, *, seed=0, tag=0, window_len=None, seq_ids=None,
                  base_pos=None, return_probs=False, ws=None, out=None, part=None, early_exit=False):
    """Stochastic window verification: sv_verify_window, one half of it
    (sv_verify_window_part) when part is SV_PART_ROW_STATS / SV_PART_DECIDE_SAMPLE,
    or sv_verify_window_early_exit when early_exit is set."""
    B, rows, V = target.shape
    gamma = rows - 1
    ts = _logits(target, gamma + 1, "target")
    ds = _logits(draft, gamma, "draft")
    if draft.dtype != target.dtype or draft.shape[0] != B or draft.shape[2] != V:
        raise ValueError("draft must match target in dtype, batch and vocabulary")
    _i32(tokens, (B, gamma), "tokens")
    _optional(window_len, torch.int32, B, "window_len")
    _optional(seq_ids, torch.int64, B, "seq_ids")
    _optional(base_pos, torch.int64, B, "base_pos")
    dev = target.device
    _same_device(dev, draft=draft, tokens=tokens, window_len=window_len, seq_ids=seq_ids,
                 base_pos=base_pos)
    if ws is None:
        ws = workspace(SV_OP_WINDOW, B, gamma, V, target.dtype, dev)
        ws_bytes = ws.numel()
    else:
        ws_bytes = _ws_bytes(ws, dev)
    if out is None:
        out = WindowResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(B, gamma + 1, dtype=torch.int32, device=dev))
        if return_probs:
            out.p_draft = torch.empty(B, gamma, dtype=torch.float32, device=dev)
            out.q_draft = torch.empty(B, gamma, dtype=torch.float32, device=dev)
    else:
        _check_window_out(out, B, gamma, dev)
    if early_exit:
        if part is not None:
            raise ValueError("early_exit has no parts")
        head = (lib().sv_verify_window_early_exit,)
    else:
        head = (lib().sv_verify_window,) if part is None else (lib().sv_verify_window_part, part)
    with torch.cuda.device(dev):
        _check(head[0](
            *head[1:], _ptr(target), ts, _ptr(draft), ds, _DTYPE_CODE[target.dtype],
            _ptr(tokens), _ptr(window_len), B, gamma, V,
            ctypes.c_uint64(seed), ctypes.c_uint64(tag), _ptr(seq_ids), _ptr(base_pos),
            _ptr(out.n_accepted), _ptr(out.out_tokens), _ptr(out.p_draft), _ptr(out.q_draft),
            _ptr(ws), ws_bytes, _stream(dev)))
    return out


def verify_window_noalloc(target, draft, tokens, *, seed=0, tag=0, window_len=None, seq_ids=None,
                          base_pos=None, return_probs=False, out=None):
    """sv_verify_window_noalloc: the stochastic window on the library's static
    per-GPU scratch, with no workspace.  Calls on one GPU must not overlap."""
    B, rows, V = target.shape
    gamma = rows - 1
    ts = _logits(target, gamma + 1, "target")
    ds = _logits(draft, gamma, "draft")
    if draft.dtype != target.dtype or draft.shape[0] != B or draft.shape[2] != V:
        raise ValueError("draft must match target in dtype, batch and vocabulary")
    _i32(tokens, (B, gamma), "tokens")
    _optional(window_len, torch.int32, B, "window_len")
    _optional(seq_ids, torch.int64, B, "seq_ids")
    _optional(base_pos, torch.int64, B, "base_pos")
    dev = target.device
    _same_device(dev, draft=draft, tokens=tokens, window_len=window_len, seq_ids=seq_ids,
                 base_pos=base_pos)
    if out is None:
        out = WindowResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(B, gamma + 1, dtype=torch.int32, device=dev))
        if return_probs:
            out.p_draft = torch.empty(B, gamma, dtype=torch.float32, device=dev)
            out.q_draft = torch.empty(B, gamma, dtype=torch.float32, device=dev)
    else:
        _check_window_out(out, B, gamma, dev)
    with torch.cuda.device(dev):
        _check(lib().sv_verify_window_noalloc(
            _ptr(target), ts, _ptr(draft), ds, _DTYPE_CODE[target.dtype],
            _ptr(tokens), _ptr(window_len), B, gamma, V,
            ctypes.c_uint64(seed), ctypes.c_uint64(tag), _ptr(seq_ids), _ptr(base_pos),
            _ptr(out.n_accepted), _ptr(out.out_tokens), _ptr(out.p_draft), _ptr(out.q_draft),
            _stream(dev)))
    return out


def verify_window_lmhead(h_target, w_target, h_draft, w_draft, tokens, *, seed=0, tag=0,
                         window_len=None, seq_ids=None, base_pos=None, return_probs=False, ws=None):
    """Window verification on logits from hidden states, LM head fused:
    sv_verify_window_lmhead.  h_target (B, gamma+1, Ht), w_target (V, Ht),
    h_draft (B, gamma, Hd), w_draft (V, Hd), all bf16 and contiguous."""
    B, rows, Ht = h_target.shape
    gamma = rows - 1
    V = w_target.shape[0]
    for name, t in (("h_target", h_target), ("w_target", w_target), ("h_draft", h_draft),
                    ("w_draft", w_draft)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous bf16 device tensor")
    Hd = h_draft.shape[2]
    if h_draft.shape[:2] != (B, gamma) or w_target.shape != (V, Ht) or w_draft.shape != (V, Hd):
        raise ValueError("hidden / unembedding shapes do not agree")
    _i32(tokens, (B, gamma), "tokens")
    _optional(window_len, torch.int32, B, "window_len")
    _optional(seq_ids, torch.int64, B, "seq_ids")
    _optional(base_pos, torch.int64, B, "base_pos")
    dev = h_target.device
    _same_device(dev, w_target=w_target, h_draft=h_draft, w_draft=w_draft, tokens=tokens,
                 window_len=window_len, seq_ids=seq_ids, base_pos=base_pos)
    if ws is None:
        ws = workspace(SV_OP_LMHEAD, B, gamma, V, torch.bfloat16, dev)
        ws_bytes = ws.numel()
    else:
        ws_bytes = _ws_bytes(ws, dev)
    out = WindowResult(torch.empty(B, dtype=torch.int32, device=dev),
                       torch.empty(B, gamma + 1, dtype=torch.int32, device=dev))
    if return_probs:
        out.p_draft = torch.empty(B, gamma, dtype=torch.float32, device=dev)
        out.q_draft = torch.empty(B, gamma, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(lib().sv_verify_window_lmhead(
            _ptr(h_target), _ptr(w_target), Ht, _ptr(h_draft), _ptr(w_draft), Hd,
            _ptr(tokens), _ptr(window_len), B, gamma, V,
            ctypes.c_uint64(seed), ctypes.c_uint64(tag), _ptr(seq_ids), _ptr(base_pos),
            _ptr(out.n_accepted), _ptr(out.out_tokens), _ptr(out.p_draft), _ptr(out.q_draft),
            _ptr(ws), ws_bytes, _stream(dev)))
    return out


def verify_greedy(target, tokens, *, window_len=None, ws=None, out=None):
    """Greedy window verification: sv_verify_greedy."""
    B, rows, V = target.shape
    gamma = rows - 1
    ts = _logits(target, gamma + 1, "target")
    _i32(tokens, (B, gamma), "tokens")
    _optional(window_len, torch.int32, B, "window_len")
    dev = target.device
    _same_device(dev, tokens=tokens, window_len=window_len)
    if ws is None:
        ws = workspace(SV_OP_GREEDY, B, gamma, V, target.dtype, dev)
        ws_bytes = ws.numel()
    else:
        ws_bytes = _ws_bytes(ws, dev)
    if out is None:
        out = WindowResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty(B, gamma + 1, dtype=torch.int32, device=dev))
    else:
        if out.n_accepted is None or out.out_tokens is None:
            raise ValueError("n_accepted and out_tokens are required outputs")
        _out_tensor(out.n_accepted, torch.int32, (B,), dev, "n_accepted")
        _out_tensor(out.out_tokens, torch.int32, (B, gamma + 1), dev, "out_tokens")
    with torch.cuda.device(dev):
        _check(lib().sv_verify_greedy(
            _ptr(target), ts, _DTYPE_CODE[target.dtype], _ptr(tokens), _ptr(window_len),
            B, gamma, V, _ptr(out.n_accepted), _ptr(out.out_tokens),
            _ptr(ws), ws_bytes, _stream(dev)))
    return out


def tree_max_depth(parent):
    arr = (ctypes.c_int32 * len(parent))(*parent)
    d = lib().sv_tree_max_depth(arr, len(parent))
    if d < 0:
        raise SvError(d)
    return d


def verify_tree(target, draft, node_tokens, parent, *, mode="stochastic", seed=0, tag=0,
                seq_ids=None, base_pos=None, ws=None):
    """Token-tree verification: sv_verify_tree.  parent is a host sequence;
    mode "greedy", "stochastic" or "multi_candidate"."""
    B, N, V = target.shape
    if len(parent) != N:
        raise ValueError("parent must have one entry per tree node")
    if target.stride(2) != 1 or target.stride(1) != V or target.stride(0) != N * V:
        raise ValueError("target must be contiguous (B, N, V)")
    if mode not in _TREE_MODES:
        raise ValueError(f"unknown tree mode {mode!r}")
    code = _TREE_MODES[mode]
    sampled = code != SV_TREE_GREEDY
    if sampled:
        if draft is None or draft.shape != target.shape or draft.dtype != target.dtype \
                or not draft.is_contiguous():
            raise ValueError("sampled modes need contiguous draft logits shaped like target")
    _i32(node_tokens, (B, N), "node_tokens")
    _optional(seq_ids, torch.int64, B, "seq_ids")
    _optional(base_pos, torch.int64, B, "base_pos")
    D = tree_max_depth(parent)
    dev = target.device
    if not target.is_cuda or target.dtype not in _DTYPE_CODE:
        raise ValueError("target: expected float32, bfloat16 or float16 device logits")
    _same_device(dev, draft=draft if sampled else None, node_tokens=node_tokens, seq_ids=seq_ids,
                 base_pos=base_pos)
    if ws is None:
        ws = workspace(SV_OP_TREE, B, N, V, target.dtype, dev)
        ws_bytes = ws.numel()
    else:
        ws_bytes = _ws_bytes(ws, dev)
    res = TreeResult(torch.empty(B, dtype=torch.int32, device=dev),
                     torch.empty(B, dtype=torch.int32, device=dev),
                     torch.empty(B, D + 1, dtype=torch.int32, device=dev),
                     torch.empty(B, max(D, 1), dtype=torch.int32, device=dev)[:, :D])
    par = (ctypes.c_int32 * N)(*parent)
    with torch.cuda.device(dev):
        _check(lib().sv_verify_tree(
            _ptr(target), _ptr(draft if sampled else None),
            _DTYPE_CODE[target.dtype], _ptr(node_tokens), par, B, N, V, code,
            ctypes.c_uint64(seed), ctypes.c_uint64(tag), _ptr(seq_ids), _ptr(base_pos),
            _ptr(res.n_accepted), _ptr(res.best_node), _ptr(res.out_tokens), _ptr(res.out_nodes),
            _ptr(ws), ws_bytes, _stream(dev)))
    return res


def rollback(buf_tokens, buf_len, stage, verified, verified_len, *, len_offset=0):
    """Per-stage buffer rollback: sv_rollback (in place on buf_tokens/buf_len).
    Row s of `verified` must hold at least verified_len[s] + len_offset tokens
    (at most cap are read); that length lives on the device and is not checked here."""
    S, K, cap = buf_tokens.shape
    _i32(buf_tokens, (S, K, cap), "buf_tokens")
    _i32(buf_len, (S, K), "buf_len")
    if verified.dtype != torch.int32 or not verified.is_cuda or verified.dim() != 2 \
            or verified.shape[0] != S or verified.stride(1) != 1:
        raise ValueError("verified: expected an int32 device tensor (S, >=L) with unit column stride")
    _i32(verified_len, (S,), "verified_len")
    dev = buf_tokens.device
    _same_device(dev, buf_len=buf_len, verified=verified, verified_len=verified_len)
    with torch.cuda.device(dev):
        _check(lib().sv_rollback(
            _ptr(buf_tokens), _ptr(buf_len), S, K, cap, stage,
            _ptr(verified), verified.stride(0), _ptr(verified_len), len_offset, _stream(dev)))


def probe_read(buf, sink=None):
    """Streams buf through the library's read-bandwidth probe kernel.  buf is
    read as one contiguous byte range; sink takes one 32-bit word per
    workgroup (sv_probe_blocks of the byte count)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf: expected a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    nb = int(lib().sv_probe_blocks(nbytes))
    if sink is None:
        sink = torch.empty(nb, dtype=torch.int32, device=buf.device)
    elif (sink.dtype not in (torch.int32, torch.uint32) or sink.device != buf.device
          or not sink.is_contiguous() or sink.numel() < nb):
        raise ValueError(f"sink: expected a contiguous 32-bit tensor of at least {nb} entries on {buf.device}")
    with torch.cuda.device(buf.device):
        _check(lib().sv_probe_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf.device)))
    return sink
