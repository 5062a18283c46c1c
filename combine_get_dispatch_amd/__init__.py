"""Python binding of libep.so: MoE expert-parallel dispatch / combine on one
MI355X (gfx950).

Argument marshalling only.  Every step of the path (layout, dispatch,
combine) runs in the HIP kernels of libep.so; torch provides device memory
and the current stream.  The raw functions below carry the C names of
include/ep.h and take preallocated torch tensors; ``EpBuffers`` allocates
the tensors for one configuration and chains the three calls.

There is no fallback: if libep.so is missing or cannot be loaded, every call
raises.  Build it with ``python -m combine_get_dispatch_amd._build``.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libep.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "ep.h")
HEADER_PATHS = [HEADER_PATH, os.path.join(os.path.dirname(_PKG), "include", "ep_probe.h")]

(EP_OK, EP_ERR_INVALID_ARG, EP_ERR_INVALID_ROUTE, EP_ERR_CAPACITY, EP_ERR_WORKSPACE, EP_ERR_HIP,
 EP_ERR_NONFINITE) = range(7)
EP_STATUS_BIT_ROUTE, EP_STATUS_BIT_CAPACITY, EP_STATUS_BIT_WORKSPACE, EP_STATUS_BIT_NONFINITE = (
    0x1, 0x2, 0x4, 0x8)
EP_DTYPE_BF16, EP_DTYPE_FP8_E4M3 = 0, 1


class EpError(RuntimeError):
    """A libep call returned a non-OK status."""

    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func}: status {status}: {message}")
        self.status = status


class ep_config_t(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32), ("expert_alignment", ctypes.c_int32)]


class ep_handle_t(ctypes.Structure):
    _fields_ = [("config", ep_config_t), ("capacity", ctypes.c_int64),
                ("tok_slot_row", ctypes.c_void_p), ("row_src", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p)]


class ep_ranked_handle_t(ctypes.Structure):
    _fields_ = [("config", ep_config_t), ("capacity", ctypes.c_int64),
                ("ranked_capacity", ctypes.c_int64), ("rank_token_offsets", ctypes.c_void_p),
                ("tok_rank_row", ctypes.c_void_p), ("tok_slot_row", ctypes.c_void_p),
                ("ne_topk_idx", ctypes.c_void_p), ("ne_topk_weights", ctypes.c_void_p),
                ("ne_src", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libep.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m combine_get_dispatch_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    P, S, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    cfgp = ctypes.POINTER(ep_config_t)
    L.ep_status_string.restype = ctypes.c_char_p
    L.ep_status_string.argtypes = [ctypes.c_int]
    for f in ("ep_last_error", "ep_last_error_string"):
        getattr(L, f).restype = ctypes.c_char_p
        getattr(L, f).argtypes = []
    L.ep_layout_workspace_bytes.argtypes = [cfgp, ctypes.POINTER(S)]
    L.ep_recv_capacity_rows.argtypes = [cfgp, ctypes.POINTER(i64)]
    L.ep_get_dispatch_layout.argtypes = [cfgp, P, P, P, P, P, P, P, S, P,
                                         ctypes.POINTER(ctypes.c_int32), P]
    i32 = ctypes.c_int32
    L.ep_dispatch.argtypes = [cfgp, ctypes.c_int, P, P, P, P, P, S, i64, i32, P, P, P, P, P, P,
                              ctypes.POINTER(ep_handle_t), P]
    L.ep_layout_dispatch.argtypes = [cfgp, ctypes.c_int, P, P, P, P, P, P, P, P, P, S, i64, i32, P,
                                     P, P, P, P, P, ctypes.POINTER(ep_handle_t), P]
    L.ep_combine.argtypes = [ctypes.POINTER(ep_handle_t), P, P, P, P]
    L.ep_read_status.argtypes = [P, P]
    L.ep_workspace_init.argtypes = [P, S, P]
    L.ep_dispatch_backward.argtypes = [ctypes.POINTER(ep_handle_t), P, P, P]
    L.ep_dispatch_fp8_input.argtypes = [cfgp, P, P, P, P, P, P, S, i64, i32, P, P, P, P, P, P,
                                        ctypes.POINTER(ep_handle_t), P]
    L.ep_layout_dispatch_noalloc.argtypes = [cfgp, ctypes.c_int, P, P, P, P, P, P, P, P, i64,
                                             i32, P, P, P, P, P, P, ctypes.POINTER(ep_handle_t),
                                             P]
    rhp = ctypes.POINTER(ep_ranked_handle_t)
    L.ep_ranked_capacity_rows.argtypes = [cfgp, ctypes.POINTER(i64)]
    L.ep_dispatch_ranked.argtypes = [cfgp, ctypes.c_int, P, P, P, P, P, S, i64, i64, P, P, P, P,
                                     P, P, P, P, P, rhp, P]
    L.ep_expand.argtypes = [rhp, ctypes.c_int, P, P, P, P, S, i32, P, P, P, P, P,
                            ctypes.POINTER(ep_handle_t), P]
    L.ep_combine_ranked.argtypes = [rhp, P, ctypes.c_int32, P, P, P]
    L.ep_combine_backward.argtypes = [ctypes.POINTER(ep_handle_t), P, P, P, P, P, P]
    L.ep_hbm_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, S, P]
    L.ep_time_next_kernel.argtypes = [P, P]
    for f in ("ep_layout_workspace_bytes", "ep_recv_capacity_rows", "ep_get_dispatch_layout",
              "ep_dispatch", "ep_layout_dispatch", "ep_combine", "ep_read_status",
              "ep_workspace_init",
              "ep_dispatch_backward", "ep_combine_backward", "ep_dispatch_fp8_input",
              "ep_ranked_capacity_rows", "ep_dispatch_ranked", "ep_expand", "ep_combine_ranked",
              "ep_hbm_probe", "ep_time_next_kernel", "ep_layout_dispatch_noalloc"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions the headers in include/ declare."""
    names = []
    for path in HEADER_PATHS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(ep_[a-z_]+)\s*\(", text)
    return names


def _check(status: int, func: str):
    if status != EP_OK:
        msg = lib().ep_last_error_string().decode()
        raise EpError(status, func, msg)


def _cfg(T, H, k, E, R, A) -> ep_config_t:
    return ep_config_t(T, H, k, E, R, A)


_current_stream = None


def _current_stream_getter():
    """A function returning torch's current stream handle on the current
    device.  torch's raw getter is used when present: building a Stream
    object per call (torch.cuda.current_stream()) costs about as much as a
    kernel launch."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    device = getattr(torch._C, "_cuda_getDevice", None)
    if raw is not None and device is not None:
        return lambda: raw(device())
    return lambda: torch.cuda.current_stream().cuda_stream


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    global _current_stream
    if _current_stream is None:
        _current_stream = _current_stream_getter()
    return ctypes.c_void_p(_current_stream())


def _ptr(t, dtype=None, shape=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


# --------------------------------------------------------------------------
# C entry points, same names as include/ep.h
# --------------------------------------------------------------------------

def ep_layout_workspace_bytes(cfg: ep_config_t) -> int:
    n = ctypes.c_size_t()
    _check(lib().ep_layout_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "ep_layout_workspace_bytes")
    return n.value


def ep_workspace_init(workspace, stream=None):
    import torch

    _check(lib().ep_workspace_init(_ptr(workspace, torch.uint8, name="workspace"),
                                   workspace.numel(), _stream(stream)), "ep_workspace_init")


def ep_recv_capacity_rows(cfg: ep_config_t) -> int:
    n = ctypes.c_int64()
    _check(lib().ep_recv_capacity_rows(ctypes.byref(cfg), ctypes.byref(n)), "ep_recv_capacity_rows")
    return n.value


def ep_get_dispatch_layout(cfg, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                           is_token_in_rank, expert_offsets, rank_offsets, workspace, status,
                           sync: bool = False, stream=None):
    """Enqueue the layout.  With sync=True, wait and return the rows used
    (raises on a device-detected error)."""
    import torch

    T, k, E, R = cfg.num_tokens, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    rows = ctypes.c_int32(-1)
    st = lib().ep_get_dispatch_layout(
        ctypes.byref(cfg), _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(num_tokens_per_rank, torch.int32, (R,), "num_tokens_per_rank"),
        _ptr(num_tokens_per_expert, torch.int32, (E,), "num_tokens_per_expert"),
        _ptr(is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(rank_offsets, torch.int32, (R + 1,), "rank_offsets"),
        _ptr(workspace, torch.uint8, name="workspace"),
        workspace.numel(), _ptr(status, torch.int32, (1,), "status"),
        ctypes.byref(rows) if sync else None, _stream(stream))
    _check(st, "ep_get_dispatch_layout")
    return rows.value if sync else None


def ep_dispatch(cfg, recv_dtype, x, topk_idx, topk_weights, expert_offsets, workspace,
                capacity, recv_x, recv_scales, recv_weights, tok_slot_row, row_src, status,
                stream=None, zero_padding: bool = True) -> ep_handle_t:
    import torch

    T, H, k, E = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts
    cap = int(capacity)
    fp8 = int(recv_dtype) == EP_DTYPE_FP8_E4M3
    handle = ep_handle_t()
    st = lib().ep_dispatch(
        ctypes.byref(cfg), int(recv_dtype), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), cap,
        1 if zero_padding else 0,
        _ptr(recv_x, torch.uint8 if fp8 else torch.bfloat16, (cap, H), "recv_x"),
        _ptr(recv_scales, torch.float32, (cap, H // 128), "recv_scales") if fp8 else None,
        _ptr(recv_weights, torch.float32, (cap,), "recv_weights"),
        _ptr(tok_slot_row, torch.int32, (T, k), "tok_slot_row"),
        _ptr(row_src, torch.int32, (cap,), "row_src"),
        _ptr(status, torch.int32, (1,), "status"), ctypes.byref(handle), _stream(stream))
    _check(st, "ep_dispatch")
    return handle


LAYOUT_DISPATCH_MAX_TOKENS = 256


def ep_layout_dispatch(cfg, recv_dtype, x, topk_idx, topk_weights, num_tokens_per_rank,
                       num_tokens_per_expert, is_token_in_rank, expert_offsets, rank_offsets,
                       workspace, capacity, recv_x, recv_scales, recv_weights, tok_slot_row,
                       row_src, status, stream=None, zero_padding: bool = True) -> ep_handle_t:
    """Layout and dispatch in one call (one launch up to 256 tokens)."""
    import torch

    T, H, k, E, R = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    cap = int(capacity)
    fp8 = int(recv_dtype) == EP_DTYPE_FP8_E4M3
    handle = ep_handle_t()
    st = lib().ep_layout_dispatch(
        ctypes.byref(cfg), int(recv_dtype), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(num_tokens_per_rank, torch.int32, (R,), "num_tokens_per_rank"),
        _ptr(num_tokens_per_expert, torch.int32, (E,), "num_tokens_per_expert"),
        _ptr(is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(rank_offsets, torch.int32, (R + 1,), "rank_offsets"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), cap,
        1 if zero_padding else 0,
        _ptr(recv_x, torch.uint8 if fp8 else torch.bfloat16, (cap, H), "recv_x"),
        _ptr(recv_scales, torch.float32, (cap, H // 128), "recv_scales") if fp8 else None,
        _ptr(recv_weights, torch.float32, (cap,), "recv_weights"),
        _ptr(tok_slot_row, torch.int32, (T, k), "tok_slot_row"),
        _ptr(row_src, torch.int32, (cap,), "row_src"),
        _ptr(status, torch.int32, (1,), "status"), ctypes.byref(handle), _stream(stream))
    _check(st, "ep_layout_dispatch")
    return handle


NOALLOC_SCRATCH_BYTES = 2 * 1024 * 1024


def ep_layout_dispatch_noalloc(cfg, recv_dtype, x, topk_idx, topk_weights, num_tokens_per_rank,
                               num_tokens_per_expert, is_token_in_rank, expert_offsets,
                               rank_offsets, capacity, recv_x, recv_scales, recv_weights,
                               tok_slot_row, row_src, status, stream=None,
                               zero_padding: bool = True) -> ep_handle_t:
    """Layout and dispatch with no workspace argument and no allocation (the
    library's own per-GPU scratch holds the layout's workspace)."""
    import torch

    T, H, k, E, R = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    cap = int(capacity)
    fp8 = int(recv_dtype) == EP_DTYPE_FP8_E4M3
    handle = ep_handle_t()
    st = lib().ep_layout_dispatch_noalloc(
        ctypes.byref(cfg), int(recv_dtype), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(num_tokens_per_rank, torch.int32, (R,), "num_tokens_per_rank"),
        _ptr(num_tokens_per_expert, torch.int32, (E,), "num_tokens_per_expert"),
        _ptr(is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(rank_offsets, torch.int32, (R + 1,), "rank_offsets"), cap,
        1 if zero_padding else 0,
        _ptr(recv_x, torch.uint8 if fp8 else torch.bfloat16, (cap, H), "recv_x"),
        _ptr(recv_scales, torch.float32, (cap, H // 128), "recv_scales") if fp8 else None,
        _ptr(recv_weights, torch.float32, (cap,), "recv_weights"),
        _ptr(tok_slot_row, torch.int32, (T, k), "tok_slot_row"),
        _ptr(row_src, torch.int32, (cap,), "row_src"),
        _ptr(status, torch.int32, (1,), "status"), ctypes.byref(handle), _stream(stream))
    _check(st, "ep_layout_dispatch_noalloc")
    return handle


def ep_dispatch_fp8_input(cfg, x_codes, x_scales, topk_idx, topk_weights, expert_offsets,
                          workspace, capacity, recv_x, recv_scales, recv_weights, tok_slot_row,
                          row_src, status, stream=None, zero_padding: bool = True) -> ep_handle_t:
    import torch

    T, H, k, E = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts
    cap = int(capacity)
    handle = ep_handle_t()
    st = lib().ep_dispatch_fp8_input(
        ctypes.byref(cfg), _ptr(x_codes, torch.uint8, (T, H), "x_codes"),
        _ptr(x_scales, torch.float32, (T, H // 128), "x_scales"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), cap,
        1 if zero_padding else 0, _ptr(recv_x, torch.uint8, (cap, H), "recv_x"),
        _ptr(recv_scales, torch.float32, (cap, H // 128), "recv_scales"),
        _ptr(recv_weights, torch.float32, (cap,), "recv_weights"),
        _ptr(tok_slot_row, torch.int32, (T, k), "tok_slot_row"),
        _ptr(row_src, torch.int32, (cap,), "row_src"),
        _ptr(status, torch.int32, (1,), "status"), ctypes.byref(handle), _stream(stream))
    _check(st, "ep_dispatch_fp8_input")
    return handle


def ep_combine(handle: ep_handle_t, expert_out, topk_weights, out, stream=None):
    import torch

    c = handle.config
    T, H, k, cap = c.num_tokens, c.hidden, c.num_topk, handle.capacity
    if expert_out is None or expert_out.dim() != 2 or expert_out.shape[1] != H \
            or expert_out.shape[0] < cap:
        raise ValueError(f"expert_out must be bf16 [>= {cap}, {H}]")
    if expert_out.shape[0] > 0:
        _ptr(expert_out, torch.bfloat16, name="expert_out")
    st = lib().ep_combine(ctypes.byref(handle),
                          ctypes.c_void_p(expert_out.data_ptr()) if expert_out.numel() else None,
                          _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
                          _ptr(out, torch.bfloat16, (T, H), "out"), _stream(stream))
    _check(st, "ep_combine")


def _rows_tensor(t, rows, H, name):
    import torch

    if t is None or t.dim() != 2 or t.shape[1] != H or t.shape[0] < rows:
        raise ValueError(f"{name} must be bf16 [>= {rows}, {H}]")
    if t.numel() == 0:
        return None
    return _ptr(t, torch.bfloat16, name=name)


def ep_dispatch_backward(handle: ep_handle_t, grad_recv_x, grad_x, stream=None):
    import torch

    c = handle.config
    st = lib().ep_dispatch_backward(
        ctypes.byref(handle), _rows_tensor(grad_recv_x, handle.capacity, c.hidden, "grad_recv_x"),
        _ptr(grad_x, torch.bfloat16, (c.num_tokens, c.hidden), "grad_x"), _stream(stream))
    _check(st, "ep_dispatch_backward")


def ep_combine_backward(handle: ep_handle_t, grad_out, topk_weights, expert_out, grad_expert_out,
                        grad_weights, stream=None):
    import torch

    c = handle.config
    T, H, k = c.num_tokens, c.hidden, c.num_topk
    st = lib().ep_combine_backward(
        ctypes.byref(handle), _ptr(grad_out, torch.bfloat16, (T, H), "grad_out"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        None if expert_out is None else _rows_tensor(expert_out, handle.capacity, H, "expert_out"),
        _rows_tensor(grad_expert_out, handle.capacity, H, "grad_expert_out"),
        _ptr(grad_weights, torch.float32, (T, k), "grad_weights"), _stream(stream))
    _check(st, "ep_combine_backward")


def ep_ranked_capacity_rows(cfg: ep_config_t) -> int:
    n = ctypes.c_int64()
    _check(lib().ep_ranked_capacity_rows(ctypes.byref(cfg), ctypes.byref(n)),
           "ep_ranked_capacity_rows")
    return n.value


def ep_dispatch_ranked(cfg, recv_dtype, x, topk_idx, topk_weights, expert_offsets, workspace,
                       capacity, ranked_capacity, ne_x, ne_scales, ne_topk_idx, ne_topk_weights,
                       ne_src, rank_token_offsets, tok_rank_row, tok_slot_row, status,
                       stream=None) -> ep_ranked_handle_t:
    import torch

    T, H, k, E, R = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks
    qc = int(ranked_capacity)
    fp8 = int(recv_dtype) == EP_DTYPE_FP8_E4M3
    h = ep_ranked_handle_t()
    st = lib().ep_dispatch_ranked(
        ctypes.byref(cfg), int(recv_dtype), _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
        _ptr(topk_weights, torch.float32, (T, k), "topk_weights"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), int(capacity), qc,
        _ptr(ne_x, torch.uint8 if fp8 else torch.bfloat16, (qc, H), "ne_x"),
        _ptr(ne_scales, torch.float32, (qc, H // 128), "ne_scales") if fp8 else None,
        _ptr(ne_topk_idx, torch.int32, (qc, k), "ne_topk_idx"),
        _ptr(ne_topk_weights, torch.float32, (qc, k), "ne_topk_weights"),
        _ptr(ne_src, torch.int32, (qc,), "ne_src"),
        _ptr(rank_token_offsets, torch.int32, (R + 1,), "rank_token_offsets"),
        _ptr(tok_rank_row, torch.int32, (T, R), "tok_rank_row"),
        _ptr(tok_slot_row, torch.int32, (T, k), "tok_slot_row"),
        _ptr(status, torch.int32, (1,), "status"), ctypes.byref(h), _stream(stream))
    _check(st, "ep_dispatch_ranked")
    return h


def ep_expand(ranked: ep_ranked_handle_t, recv_dtype, ne_x, ne_scales, expert_offsets, workspace,
              recv_x, recv_scales, recv_weights, row_src, status, stream=None,
              zero_padding: bool = True) -> ep_handle_t:
    import torch

    c = ranked.config
    H, E = c.hidden, c.num_experts
    qc, cap = ranked.ranked_capacity, ranked.capacity
    fp8 = int(recv_dtype) == EP_DTYPE_FP8_E4M3
    h = ep_handle_t()
    st = lib().ep_expand(
        ctypes.byref(ranked), int(recv_dtype),
        _ptr(ne_x, torch.uint8 if fp8 else torch.bfloat16, (qc, H), "ne_x"),
        _ptr(ne_scales, torch.float32, (qc, H // 128), "ne_scales") if fp8 else None,
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(workspace, torch.uint8, name="workspace"), workspace.numel(),
        1 if zero_padding else 0,
        _ptr(recv_x, torch.uint8 if fp8 else torch.bfloat16, (cap, H), "recv_x"),
        _ptr(recv_scales, torch.float32, (cap, H // 128), "recv_scales") if fp8 else None,
        _ptr(recv_weights, torch.float32, (cap,), "recv_weights"),
        _ptr(row_src, torch.int32, (cap,), "row_src"),
        _ptr(status, torch.int32, (1,), "status"), ctypes.byref(h), _stream(stream))
    _check(st, "ep_expand")
    return h


def ep_combine_ranked(ranked: ep_ranked_handle_t, expert_out, weighted: bool, partials, out,
                      stream=None):
    import torch

    c = ranked.config
    T, H = c.num_tokens, c.hidden
    st = lib().ep_combine_ranked(
        ctypes.byref(ranked), _rows_tensor(expert_out, ranked.capacity, H, "expert_out"),
        1 if weighted else 0,
        _ptr(partials, torch.float32, (ranked.ranked_capacity, H), "partials"),
        _ptr(out, torch.bfloat16, (T, H), "out"), _stream(stream))
    _check(st, "ep_combine_ranked")


def make_handle(num_tokens, hidden, num_topk, capacity, tok_slot_row, row_src=None,
                expert_offsets=None, num_experts=None, num_ranks=1, expert_alignment=1):
    """Build an ep_handle_t around existing device arrays (combine only reads
    the config, the capacity and tok_slot_row)."""
    import torch

    E = num_topk if num_experts is None else num_experts
    h = ep_handle_t()
    h.config = _cfg(num_tokens, hidden, num_topk, E, num_ranks, expert_alignment)
    h.capacity = int(capacity)
    p = _ptr(tok_slot_row, torch.int32, (num_tokens, num_topk), "tok_slot_row")
    h.tok_slot_row = p.value if p is not None else None
    h.row_src = row_src.data_ptr() if row_src is not None else None
    h.expert_offsets = expert_offsets.data_ptr() if expert_offsets is not None else None
    return h


def ep_read_status(status, stream=None):
    import torch

    _check(lib().ep_read_status(_ptr(status, torch.int32), _stream(stream)), "ep_read_status")


EP_PROBE_READ, EP_PROBE_WRITE, EP_PROBE_COPY = 0, 1, 2


def ep_hbm_probe(kind: int, nontemporal: bool, workgroups: int, src, dst, nbytes: int,
                 stream=None):
    """Enqueue one streaming read / write / copy pass over nbytes (a
    measurement aid, include/ep_probe.h)."""
    _check(lib().ep_hbm_probe(int(kind), int(bool(nontemporal)), int(workgroups),
                              None if src is None else ctypes.c_void_p(src.data_ptr()),
                              ctypes.c_void_p(dst.data_ptr()), int(nbytes), _stream(stream)),
           "ep_hbm_probe")


def ep_time_next_kernel(start, stop):
    """The calling thread's next layout, dispatch or combine kernel records
    the two torch timing events when it starts and ends (include/ep_probe.h);
    start.elapsed_time(stop) is then that kernel's own duration.  The events
    must already exist on the device (recorded once); either may be None."""
    def handle(ev):
        return None if ev is None else ctypes.c_void_p(ev.cuda_event)

    _check(lib().ep_time_next_kernel(handle(start), handle(stop)), "ep_time_next_kernel")


# --------------------------------------------------------------------------
# Buffers for one configuration
# --------------------------------------------------------------------------

class EpBuffers:
    """Device tensors for one (T, H, k, E, R, A, dtype) configuration, and
    the three calls on them.  Tensors are allocated once with torch and
    reused; outputs are views into them."""

    def __init__(self, num_tokens, hidden, num_topk, num_experts, num_ranks,
                 expert_alignment=1, fp8=False, capacity=None, device="cuda", zero_padding=True):
        import torch

        self.cfg = _cfg(num_tokens, hidden, num_topk, num_experts, num_ranks, expert_alignment)
        self.fp8 = bool(fp8)
        # alignment padding rows: zero payload and scales (True), or left as they are
        self.zero_padding = bool(zero_padding)
        self.capacity = ep_recv_capacity_rows(self.cfg) if capacity is None else int(capacity)
        T, H, k, E, R = num_tokens, hidden, num_topk, num_experts, num_ranks
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.workspace = torch.empty(ep_layout_workspace_bytes(self.cfg), dtype=torch.uint8, device=dev)
        ep_workspace_init(self.workspace)
        self.status = torch.zeros(1, **i32)
        self.num_tokens_per_rank = torch.empty(R, **i32)
        self.num_tokens_per_expert = torch.empty(E, **i32)
        self.is_token_in_rank = torch.empty((T, R), dtype=torch.uint8, device=dev)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.rank_offsets = torch.empty(R + 1, **i32)
        cap = self.capacity
        if self.fp8:
            self.recv_x = torch.empty((cap, H), dtype=torch.uint8, device=dev)
            self.recv_scales = torch.empty((cap, H // 128 if H % 128 == 0 else 1),
                                           dtype=torch.float32, device=dev)
        else:
            self.recv_x = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
            self.recv_scales = None
        self.recv_weights = torch.empty(cap, dtype=torch.float32, device=dev)
        self.tok_slot_row = torch.empty((T, k), **i32)
        self.row_src = torch.empty(cap, **i32)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.handle = None
        self._shape_tk = (T, k)
        self._shape_th = (T, H)
        self._handle_out = ep_handle_t()
        self._marshal()

    # The buffers' pointers are marshalled once (and again whenever one of
    # them is replaced); each call then checks only the caller's tensors.
    _MARSHALLED = frozenset({"num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
                             "expert_offsets", "rank_offsets", "workspace", "status", "recv_x",
                             "recv_scales", "recv_weights", "tok_slot_row", "row_src", "out",
                             "zero_padding"})

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        if name in EpBuffers._MARSHALLED and "_layout_args" in self.__dict__:
            self._marshal()

    def _marshal(self):
        import torch

        c = self.cfg
        T, H, k, E, R = c.num_tokens, c.hidden, c.num_topk, c.num_experts, c.num_ranks
        cap, i32, d = self.capacity, torch.int32, self.__dict__
        d["_cfg_ref"] = ctypes.byref(self.cfg)
        ws_bytes = self.workspace.numel()
        ws = _ptr(self.workspace, torch.uint8, name="workspace")
        offs = _ptr(self.expert_offsets, i32, (E + 1,), "expert_offsets")
        status = _ptr(self.status, i32, (1,), "status")
        d["_layout_args"] = (_ptr(self.num_tokens_per_rank, i32, (R,), "num_tokens_per_rank"),
                             _ptr(self.num_tokens_per_expert, i32, (E,), "num_tokens_per_expert"),
                             _ptr(self.is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank"),
                             offs, _ptr(self.rank_offsets, i32, (R + 1,), "rank_offsets"),
                             ws, ws_bytes, status)
        # the scales' width is left to the library, which rejects FP8 with H % 128 != 0
        d["_dispatch_args"] = (offs, ws, ws_bytes, cap, 1 if self.zero_padding else 0,
                               _ptr(self.recv_x, torch.uint8 if self.fp8 else torch.bfloat16,
                                    (cap, H), "recv_x"),
                               _ptr(self.recv_scales, torch.float32, name="recv_scales")
                               if self.fp8 else None)
        d["_dispatch_tail"] = (_ptr(self.tok_slot_row, i32, (T, k), "tok_slot_row"),
                               _ptr(self.row_src, i32, (cap,), "row_src"), status)
        d["_recv_weights_ptr"] = _ptr(self.recv_weights, torch.float32, (cap,), "recv_weights")
        d["_dtype"] = EP_DTYPE_FP8_E4M3 if self.fp8 else EP_DTYPE_BF16
        d["_out_ptr"] = _ptr(self.out, torch.bfloat16, (T, H), "out")

    def layout(self, topk_idx, sync=False, stream=None):
        import torch

        if sync:
            return ep_get_dispatch_layout(self.cfg, topk_idx, self.num_tokens_per_rank,
                                          self.num_tokens_per_expert, self.is_token_in_rank,
                                          self.expert_offsets, self.rank_offsets,
                                          self.workspace, self.status, sync=True, stream=stream)
        st = lib().ep_get_dispatch_layout(
            self._cfg_ref, _ptr(topk_idx, torch.int32, self._shape_tk, "topk_idx"),
            *self._layout_args, None, _stream(stream))
        _check(st, "ep_get_dispatch_layout")
        return None

    def dispatch(self, x, topk_idx, topk_weights, stream=None):
        import torch

        st = lib().ep_dispatch(
            self._cfg_ref, self._dtype, _ptr(x, torch.bfloat16, self._shape_th, "x"),
            _ptr(topk_idx, torch.int32, self._shape_tk, "topk_idx"),
            _ptr(topk_weights, torch.float32, self._shape_tk, "topk_weights"),
            *self._dispatch_args,
            self._recv_weights_ptr if topk_weights is not None else None,
            *self._dispatch_tail, ctypes.byref(self._handle_out), _stream(stream))
        _check(st, "ep_dispatch")
        self.handle = self._handle_out
        return self.handle

    def layout_dispatch(self, x, topk_idx, topk_weights, stream=None):
        """Layout and dispatch in one call (ep_layout_dispatch: one launch up
        to 256 tokens); leaves the same buffers, workspace and handle as
        layout() then dispatch()."""
        import torch

        la = self._layout_args
        st = lib().ep_layout_dispatch(
            self._cfg_ref, self._dtype, _ptr(x, torch.bfloat16, self._shape_th, "x"),
            _ptr(topk_idx, torch.int32, self._shape_tk, "topk_idx"),
            _ptr(topk_weights, torch.float32, self._shape_tk, "topk_weights"),
            la[0], la[1], la[2], la[3], la[4], la[5], la[6], self.capacity,
            self._dispatch_args[4], self._dispatch_args[5], self._dispatch_args[6],
            self._recv_weights_ptr if topk_weights is not None else None,
            self._dispatch_tail[0], self._dispatch_tail[1], self._dispatch_tail[2],
            ctypes.byref(self._handle_out), _stream(stream))
        _check(st, "ep_layout_dispatch")
        self.handle = self._handle_out
        return self.handle

    def layout_and_dispatch(self, x, topk_idx, topk_weights, stream=None):
        """Layout then dispatch through ep_layout_dispatch (the same results
        as the two calls)."""
        return self.layout_dispatch(x, topk_idx, topk_weights, stream=stream)

    def dispatch_fp8_input(self, x_codes, x_scales, topk_idx, topk_weights, stream=None):
        if not self.fp8:
            raise ValueError("dispatch_fp8_input needs buffers built with fp8=True")
        self.handle = ep_dispatch_fp8_input(
            self.cfg, x_codes, x_scales, topk_idx, topk_weights, self.expert_offsets,
            self.workspace, self.capacity, self.recv_x, self.recv_scales,
            self.recv_weights if topk_weights is not None else None, self.tok_slot_row,
            self.row_src, self.status, stream=stream, zero_padding=self.zero_padding)
        return self.handle

    def combine(self, expert_out, topk_weights, out=None, stream=None):
        import torch

        if out is not None or self.handle is not self._handle_out:
            out = self.out if out is None else out
            ep_combine(self.handle, expert_out, topk_weights, out, stream=stream)
            return out
        H, cap = self.cfg.hidden, self.capacity
        if expert_out is None or expert_out.dim() != 2 or expert_out.shape[1] != H \
                or expert_out.shape[0] < cap:
            raise ValueError(f"expert_out must be bf16 [>= {cap}, {H}]")
        y = _ptr(expert_out, torch.bfloat16, name="expert_out") if expert_out.numel() else None
        st = lib().ep_combine(ctypes.byref(self._handle_out), y,
                              _ptr(topk_weights, torch.float32, self._shape_tk, "topk_weights"),
                              self._out_ptr, _stream(stream))
        _check(st, "ep_combine")
        return self.out

    def dispatch_backward(self, grad_recv_x, grad_x=None, stream=None):
        import torch

        if grad_x is None:
            grad_x = torch.empty_like(self.out)
        ep_dispatch_backward(self.handle, grad_recv_x, grad_x, stream=stream)
        return grad_x

    def combine_backward(self, grad_out, topk_weights, expert_out, grad_expert_out=None,
                         grad_weights=None, stream=None):
        import torch

        if grad_expert_out is None:
            grad_expert_out = torch.empty((self.capacity, self.cfg.hidden), dtype=torch.bfloat16,
                                          device=grad_out.device)
        ep_combine_backward(self.handle, grad_out, topk_weights, expert_out, grad_expert_out,
                            grad_weights, stream=stream)
        return grad_expert_out

    # --- non-expanded (rank-deduplicated) path; its buffers are made on first use

    def _ranked_buffers(self):
        import torch

        if getattr(self, "ne_x", None) is not None:
            return
        c, dev = self.cfg, self.out.device
        T, H, k, R = c.num_tokens, c.hidden, c.num_topk, c.num_ranks
        qc = ep_ranked_capacity_rows(c)
        self.ranked_capacity = qc
        i32 = dict(dtype=torch.int32, device=dev)
        self.ne_x = torch.empty((qc, H), dtype=torch.uint8 if self.fp8 else torch.bfloat16,
                                device=dev)
        self.ne_scales = (torch.empty((qc, H // 128), dtype=torch.float32, device=dev)
                          if self.fp8 else None)
        self.ne_topk_idx = torch.empty((qc, k), **i32)
        self.ne_topk_weights = torch.empty((qc, k), dtype=torch.float32, device=dev)
        self.ne_src = torch.empty(qc, **i32)
        self.rank_token_offsets = torch.empty(R + 1, **i32)
        self.tok_rank_row = torch.empty((T, R), **i32)
        self.partials = None

    def dispatch_ranked(self, x, topk_idx, topk_weights, stream=None):
        self._ranked_buffers()
        self.ranked = ep_dispatch_ranked(
            self.cfg, EP_DTYPE_FP8_E4M3 if self.fp8 else EP_DTYPE_BF16, x, topk_idx, topk_weights,
            self.expert_offsets, self.workspace, self.capacity, self.ranked_capacity, self.ne_x,
            self.ne_scales, self.ne_topk_idx, self.ne_topk_weights, self.ne_src,
            self.rank_token_offsets, self.tok_rank_row, self.tok_slot_row, self.status,
            stream=stream)
        return self.ranked

    def expand(self, with_weights=True, stream=None):
        self.handle = ep_expand(self.ranked, EP_DTYPE_FP8_E4M3 if self.fp8 else EP_DTYPE_BF16,
                                self.ne_x, self.ne_scales, self.expert_offsets, self.workspace,
                                self.recv_x, self.recv_scales,
                                self.recv_weights if with_weights else None, self.row_src,
                                self.status, stream=stream, zero_padding=self.zero_padding)
        return self.handle

    def combine_ranked(self, expert_out, weighted=True, out=None, stream=None):
        import torch

        if self.partials is None:
            self.partials = torch.empty((self.ranked_capacity, self.cfg.hidden),
                                        dtype=torch.float32, device=self.out.device)
        out = self.out if out is None else out
        ep_combine_ranked(self.ranked, expert_out, weighted, self.partials, out, stream=stream)
        return out

    def check_status(self, stream=None):
        ep_read_status(self.status, stream=stream)
