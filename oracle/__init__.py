"""Plain CPU oracle for the MoE dispatch / combine layout transformation.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark are the only code that may import this package.  The product
path (the HIP library and its Python binding) never touches it, and the two
share no code.

The arithmetic lives in ``oracle.c`` (plain sequential C, compiled with gcc,
no fast-math, no FP contraction); this module only marshals numpy arrays to it
through ctypes.  Every function returns numpy arrays and raises
``OracleError`` with the oracle's status code on rejected input.

Sources: "GPU microarchitecture: DeepEP first principles" (sections 1.1, 1.2,
6.1, 6.2, 7.1) and "Deep Dive - DeepEP" (sections "Dispatch: layout, move, and
epilogue", "Combine: reverse routing plus reduction", "Precision: FP8 on the
wire, BF16 for the reduction", "A runnable routing ledger").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, BAD_ARG, BAD_ROUTE, NO_CAPACITY = 0, 1, 2, 3

GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
             "-fno-fast-math", "-fPIC", "-shared"]


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} rejected its input (status {code})")
        self.code = code


def build_library() -> str:
    """Compile oracle.c into liboracle.so with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # EP_ORACLE_LIB names another build of oracle.c (the mutation check,
    # tests/oracle_mutations.py, loads planted-mistake builds this way)
    path = os.environ.get("EP_ORACLE_LIB")
    if path is None:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_library()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_round.argtypes = [ctypes.c_float]
    lib.oracle_bf16_to_float.restype = ctypes.c_float
    lib.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    for name in ("oracle_bf16_round_array", "oracle_e4m3_encode_array",
                 "oracle_e4m3_value_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [i64, P, P]
    lib.oracle_layout.restype = ctypes.c_int
    lib.oracle_layout.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_dispatch.restype = ctypes.c_int
    lib.oracle_dispatch.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P,
                                    i64, P, P, P, P, P]
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [i32, i32, i32, i64, P, P, P, P, P]
    lib.oracle_dispatch_fp8_input.restype = ctypes.c_int
    lib.oracle_dispatch_fp8_input.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, i64,
                                              P, P, P, P, P]
    lib.oracle_dispatch_ranked.restype = ctypes.c_int
    lib.oracle_dispatch_ranked.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, i64,
                                           P, P, P, P, P, P, P]
    lib.oracle_expand.restype = ctypes.c_int
    lib.oracle_expand.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, i64,
                                  P, P, P, P, P]
    lib.oracle_combine_ranked.restype = ctypes.c_int
    lib.oracle_combine_ranked.argtypes = [i32, i32, i32, i32, i64, i64, i32, P, P, P, P, P,
                                          P, P, P, P]
    lib.oracle_dispatch_backward.restype = ctypes.c_int
    lib.oracle_dispatch_backward.argtypes = [i32, i32, i32, i64, P, P, P, P]
    lib.oracle_combine_backward.restype = ctypes.c_int
    lib.oracle_combine_backward.argtypes = [i32, i32, i32, i64, i64, P, P, P, P, P, P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------

def bf16_round(v) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_round_array(v.size, _ptr(v), _ptr(out))
    return out


def bf16_to_float(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    bits = _c(bits, np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(v) -> np.ndarray:
    """fp32 values -> OCP E4M3FN codes (uint8), RNE, saturating."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_encode_array(v.size, _ptr(v), _ptr(out))
    return out


def e4m3_value(codes) -> np.ndarray:
    """E4M3FN codes -> float64 values (NaN for 0x7F / 0xFF)."""
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().oracle_e4m3_value_array(codes.size, _ptr(codes), _ptr(out))
    return out


# --------------------------------------------------------------------------
# the path
# --------------------------------------------------------------------------

def layout(topk_idx, num_experts: int, num_ranks: int, alignment: int = 1) -> dict:
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    E, R = num_experts, num_ranks
    out = dict(
        num_tokens_per_rank=np.zeros(R, np.int32),
        num_tokens_per_expert=np.zeros(E, np.int32),
        is_token_in_rank=np.zeros((T, R), np.uint8),
        expert_offsets=np.zeros(E + 1, np.int32),
        rank_offsets=np.zeros(R + 1, np.int32),
    )
    rc = _load().oracle_layout(T, k, E, R, alignment, _ptr(idx),
                               _ptr(out["num_tokens_per_rank"]),
                               _ptr(out["num_tokens_per_expert"]),
                               _ptr(out["is_token_in_rank"]),
                               _ptr(out["expert_offsets"]),
                               _ptr(out["rank_offsets"]))
    if rc:
        raise OracleError(rc, "layout")
    return out


def dispatch(x_bits, topk_idx, topk_weights, num_experts: int, num_ranks: int,
             alignment: int = 1, fp8: bool = False, capacity: int | None = None,
             fill_recv: int = 0) -> dict:
    """Returns recv_x (uint16 [cap,H] or uint8 [cap,H]), recv_scales
    (fp32 [cap,H/128] or None), recv_weights, tok_slot_row, row_src.
    Rows past expert_offsets[E] keep the fill value ``fill_recv``."""
    x = _c(x_bits, np.uint16)
    idx = _c(topk_idx, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    if capacity is None:
        capacity = T * k + num_experts * (alignment - 1)
    if fp8:
        recv_x = np.full((capacity, H), fill_recv & 0xFF, np.uint8)
        recv_scales = np.zeros((capacity, H // 128 if H % 128 == 0 else 1), np.float32)
    else:
        recv_x = np.full((capacity, H), fill_recv & 0xFFFF, np.uint16)
        recv_scales = None
    recv_weights = np.zeros(capacity, np.float32) if w is not None else None
    tok_slot_row = np.zeros((T, k), np.int32)
    row_src = np.full(capacity, -2, np.int32)
    rc = _load().oracle_dispatch(T, H, k, num_experts, num_ranks, alignment,
                                 1 if fp8 else 0, _ptr(x), _ptr(idx), _ptr(w),
                                 capacity, _ptr(recv_x), _ptr(recv_scales),
                                 _ptr(recv_weights), _ptr(tok_slot_row),
                                 _ptr(row_src))
    if rc:
        raise OracleError(rc, "dispatch")
    return dict(recv_x=recv_x, recv_scales=recv_scales, recv_weights=recv_weights,
                tok_slot_row=tok_slot_row, row_src=row_src)


def dispatch_fp8_input(codes, scales, topk_idx, topk_weights, num_experts: int, num_ranks: int,
                       alignment: int = 1, capacity: int | None = None,
                       fill_recv: int = 0) -> dict:
    """Dispatch of pre-quantised rows: E4M3 codes (uint8 [T,H]) and fp32
    scales [T,H/128] copied to the receive rows."""
    q = _c(codes, np.uint8)
    sc = _c(scales, np.float32)
    idx = _c(topk_idx, np.int32)
    T, H = q.shape
    k = idx.shape[1]
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    if capacity is None:
        capacity = T * k + num_experts * (alignment - 1)
    recv_x = np.full((capacity, H), fill_recv & 0xFF, np.uint8)
    recv_scales = np.zeros((capacity, max(H // 128, 1)), np.float32)
    recv_weights = np.zeros(capacity, np.float32) if w is not None else None
    tok_slot_row = np.zeros((T, k), np.int32)
    row_src = np.full(capacity, -2, np.int32)
    rc = _load().oracle_dispatch_fp8_input(T, H, k, num_experts, num_ranks, alignment, _ptr(q),
                                           _ptr(sc), _ptr(idx), _ptr(w), capacity,
                                           _ptr(recv_x), _ptr(recv_scales), _ptr(recv_weights),
                                           _ptr(tok_slot_row), _ptr(row_src))
    if rc:
        raise OracleError(rc, "dispatch_fp8_input")
    return dict(recv_x=recv_x, recv_scales=recv_scales, recv_weights=recv_weights,
                tok_slot_row=tok_slot_row, row_src=row_src)


def combine(y_bits, tok_slot_row, topk_weights) -> tuple[np.ndarray, np.ndarray]:
    """Returns (out bf16 bits uint16 [T,H], fp32 accumulator [T,H])."""
    y = _c(y_bits, np.uint16)
    tsr = _c(tok_slot_row, np.int32)
    cap, H = y.shape
    T, k = tsr.shape
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    out = np.empty((T, H), np.uint16)
    acc = np.empty((T, H), np.float32)
    rc = _load().oracle_combine(T, H, k, cap, _ptr(y), _ptr(tsr), _ptr(w),
                                _ptr(out), _ptr(acc))
    if rc:
        raise OracleError(rc, "combine")
    return out, acc


def dispatch_backward(grad_recv_bits, tok_slot_row) -> tuple[np.ndarray, np.ndarray]:
    """Transpose of the unweighted dispatch: returns (grad_x bf16 bits
    [T,H], fp32 accumulator [T,H])."""
    g = _c(grad_recv_bits, np.uint16)
    tsr = _c(tok_slot_row, np.int32)
    cap, H = g.shape
    T, k = tsr.shape
    out = np.empty((T, H), np.uint16)
    acc = np.empty((T, H), np.float32)
    rc = _load().oracle_dispatch_backward(T, H, k, cap, _ptr(g), _ptr(tsr), _ptr(out), _ptr(acc))
    if rc:
        raise OracleError(rc, "dispatch_backward")
    return out, acc


def combine_backward(grad_out_bits, tok_slot_row, topk_weights, expert_out_bits, rows_used: int,
                     capacity: int | None = None, fill: int = 0) -> dict:
    """Backward of combine: grad_expert_out (bf16 bits [cap,H]; rows past
    rows_used keep ``fill``), grad_w and grad_w_abs (fp64 [T,k]; None when
    expert_out_bits is None)."""
    g = _c(grad_out_bits, np.uint16)
    tsr = _c(tok_slot_row, np.int32)
    T, H = g.shape
    k = tsr.shape[1]
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    y = None if expert_out_bits is None else _c(expert_out_bits, np.uint16)
    cap = rows_used if capacity is None else capacity
    gy = np.full((cap, H), fill & 0xFFFF, np.uint16)
    gw = np.zeros((T, k), np.float64) if y is not None else None
    ga = np.zeros((T, k), np.float64) if y is not None else None
    rc = _load().oracle_combine_backward(T, H, k, cap, rows_used, _ptr(g), _ptr(tsr), _ptr(w),
                                         _ptr(y), _ptr(gy), _ptr(gw), _ptr(ga))
    if rc:
        raise OracleError(rc, "combine_backward")
    return dict(grad_expert_out=gy, grad_w=gw, grad_w_abs=ga)


def dispatch_ranked(x_bits, topk_idx, topk_weights, num_experts: int, num_ranks: int,
                    fp8: bool = False, capacity: int | None = None) -> dict:
    """Non-expanded dispatch: one row per (token, destination rank)."""
    x = _c(x_bits, np.uint16)
    idx = _c(topk_idx, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    R = num_ranks
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    if capacity is None:
        capacity = T * min(k, R)
    rto = np.zeros(R + 1, np.int32)
    if fp8:
        recv_x = np.zeros((capacity, H), np.uint8)
        recv_scales = np.zeros((capacity, max(H // 128, 1)), np.float32)
    else:
        recv_x = np.zeros((capacity, H), np.uint16)
        recv_scales = None
    rti = np.full((capacity, k), -2, np.int32)
    rtw = np.zeros((capacity, k), np.float32)
    src = np.full(capacity, -2, np.int32)
    trr = np.zeros((T, R), np.int32)
    rc = _load().oracle_dispatch_ranked(T, H, k, num_experts, R, 1 if fp8 else 0, _ptr(x),
                                        _ptr(idx), _ptr(w), capacity, _ptr(rto), _ptr(recv_x),
                                        _ptr(recv_scales), _ptr(rti), _ptr(rtw), _ptr(src),
                                        _ptr(trr))
    if rc:
        raise OracleError(rc, "dispatch_ranked")
    return dict(rank_token_offsets=rto, recv_x=recv_x, recv_scales=recv_scales,
                recv_topk_idx=rti, recv_topk_weights=rtw, recv_src=src, tok_rank_row=trr)


def expand(ne: dict, T: int, k: int, num_experts: int, num_ranks: int, alignment: int = 1,
           fp8: bool = False, capacity: int | None = None) -> dict:
    """Receiver-side expand of dispatch_ranked's rows into the expert-major
    layout (same outputs as dispatch)."""
    H = ne["recv_x"].shape[1]
    if capacity is None:
        capacity = T * k + num_experts * (alignment - 1)
    recv_x = np.zeros((capacity, H), np.uint8 if fp8 else np.uint16)
    recv_scales = np.zeros((capacity, max(H // 128, 1)), np.float32) if fp8 else None
    recv_weights = np.zeros(capacity, np.float32)
    tsr = np.zeros((T, k), np.int32)
    row_src = np.full(capacity, -2, np.int32)
    rc = _load().oracle_expand(T, H, k, num_experts, num_ranks, alignment, 1 if fp8 else 0,
                               _ptr(_c(ne["rank_token_offsets"], np.int32)),
                               _ptr(np.ascontiguousarray(ne["recv_x"])),
                               _ptr(None if ne["recv_scales"] is None
                                    else _c(ne["recv_scales"], np.float32)),
                               _ptr(_c(ne["recv_topk_idx"], np.int32)),
                               _ptr(_c(ne["recv_topk_weights"], np.float32)),
                               _ptr(_c(ne["recv_src"], np.int32)), capacity, _ptr(recv_x),
                               _ptr(recv_scales), _ptr(recv_weights), _ptr(tsr), _ptr(row_src))
    if rc:
        raise OracleError(rc, "expand")
    return dict(recv_x=recv_x, recv_scales=recv_scales, recv_weights=recv_weights,
                tok_slot_row=tsr, row_src=row_src)


def combine_ranked(y_bits, tok_slot_row, ne: dict, weighted: bool = True):
    """Combine through per-rank fp32 partials: returns (out bf16 bits [T,H],
    stage-2 fp32 accumulator [T,H], partials fp32 [rows,H])."""
    y = _c(y_bits, np.uint16)
    tsr = _c(tok_slot_row, np.int32)
    cap, H = y.shape
    T, k = tsr.shape
    trr = _c(ne["tok_rank_row"], np.int32)
    R = trr.shape[1]
    rows = int(ne["rank_token_offsets"][-1])
    part = np.zeros((max(rows, 1), H), np.float32)
    out = np.empty((T, H), np.uint16)
    acc = np.empty((T, H), np.float32)
    rc = _load().oracle_combine_ranked(T, H, k, R, rows, cap, 1 if weighted else 0, _ptr(y),
                                       _ptr(tsr), _ptr(_c(ne["recv_topk_idx"], np.int32)),
                                       _ptr(_c(ne["recv_topk_weights"], np.float32)),
                                       _ptr(_c(ne["recv_src"], np.int32)), _ptr(trr),
                                       _ptr(part), _ptr(out), _ptr(acc))
    if rc:
        raise OracleError(rc, "combine_ranked")
    return out, acc, part[:rows]
