"""Worked examples from the pages, written once and run through any backend.

A backend is an object with numpy-in / numpy-out methods

    layout(topk_idx, E, R, A) -> dict(num_tokens_per_rank, num_tokens_per_expert,
                                      is_token_in_rank, expert_offsets, rank_offsets)
    dispatch(x_bits, topk_idx, topk_weights, E, R, A, fp8, capacity) -> dict(
        recv_x, recv_scales, recv_weights, tok_slot_row, row_src)
    combine(y_bits, tok_slot_row, topk_weights) -> out bits [T,H] (uint16)

and an attribute ``hidden_multiple`` (the hidden size must be a multiple of
it; rows are zero-padded up to it).  The oracle backend and the HIP backend
both satisfy it, so every page example pins the oracle on the CPU and is then
replayed against the GPU path.
"""
from __future__ import annotations

import numpy as np

from tests.golden_fixtures import load


def bf16_bits_exact(vals) -> np.ndarray:
    """Values that bf16 represents exactly -> bit patterns (asserts exactness)."""
    f = np.ascontiguousarray(vals, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, f), "value not exactly representable in bf16"
    return bits


def bits_to_f32(bits) -> np.ndarray:
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def row_experts(expert_offsets: np.ndarray, rows: int) -> np.ndarray:
    """Expert that owns each receive row (segment lookup)."""
    p = np.arange(rows)
    return np.searchsorted(expert_offsets, p, side="right") - 1


def _pad(H: int, mult: int) -> int:
    return ((H + mult - 1) // mult) * mult


class Ledger:
    """The four-token ledger ("Deep Dive - DeepEP", "A runnable routing ledger")."""

    def __init__(self):
        self.fx = load("four_token_ledger.txt")
        self.var = load("ledger_variants.txt")
        self.tokens = self.fx["tokens"]
        self.E = self.fx.num("num_experts", int)
        self.R = self.fx.num("num_ranks", int)
        self.hidden = np.array([self.fx.nums(f"hidden.{t}") for t in self.tokens], np.float32)

    def routes(self, override: dict | None = None):
        idx, w = [], []
        for t in self.tokens:
            vals = self.fx[f"route.{t}"]
            if override and t in override:
                vals = override[t]
            idx.append([int(vals[0]), int(vals[2])])
            w.append([float(vals[1]), float(vals[3])])
        return np.array(idx, np.int32), np.array(w, np.float32)

    def run(self, be, idx, w, alignment=1, weighting="combine"):
        """Dispatch, apply the toy experts (expert e multiplies by e+1), then
        combine.  weighting: "combine" (raw rows, combine applies the gate),
        "caller" (rows pre-weighted, combine sums), "none" (raw rows, summed),
        "twice" (pre-weighted rows and combine applies the gate again)."""
        T, H = self.hidden.shape
        Hp = _pad(H, be.hidden_multiple)
        x = np.zeros((T, Hp), np.float32)
        x[:, :H] = self.hidden
        xb = bf16_bits_exact(x)
        lay = be.layout(idx, self.E, self.R, alignment)
        cap = T * idx.shape[1] + self.E * (alignment - 1)
        d = be.dispatch(xb, idx, w, self.E, self.R, alignment, False, cap)
        used = int(lay["expert_offsets"][-1])
        rexp = row_experts(lay["expert_offsets"], used)
        y = np.zeros((cap, Hp), np.float32)
        for p in range(used):
            src = int(d["row_src"][p])
            if src < 0:
                continue
            t, j = divmod(src, idx.shape[1])
            raw = (rexp[p] + 1) * bits_to_f32(d["recv_x"][p])
            if weighting in ("caller", "twice"):
                raw = np.float32(d["recv_weights"][p]) * raw
            y[p] = raw
        yb = bf16_bits_exact(y) if weighting in ("combine", "none") else _round_bf16_np(y)
        cw = w if weighting in ("combine", "twice") else None
        out = be.combine(yb, d["tok_slot_row"], cw)
        return dict(layout=lay, dispatch=d, out=bits_to_f32(out)[:, :H], rows_used=used,
                    row_expert=rexp)


def _round_bf16_np(v):
    """bf16 rounding of caller-side (test-side) expert outputs, done with
    torch's own conversion so the test does not reuse the oracle's."""
    from ep_workloads import to_bf16_bits

    return to_bf16_bits(v)
