"""Pins for the oracle's backward functions (CPU only): the ledger's hand
gradients, fp64 adjoint identities, a finite-difference check of the gate
gradient through the forward combine, brute force on tiny inputs, and the
transpose duality between dispatch and combine for unweighted routes."""
import numpy as np
import pytest
import torch

import oracle
from ep_workloads import random_routes
from tests.ep_cases import Ledger, bf16_bits_exact, bits_to_f32, row_experts


def _rand_bf16(rng, shape, scale=1.0):
    return (np.asarray(rng.standard_normal(shape) * scale, np.float32).view(np.uint32)
            >> 16).astype(np.uint16)


def test_ledger_gradients(golden):
    fx = golden("ledger_gradients.txt")
    L = Ledger()
    idx, w = L.routes()
    r = L.run(_OracleBE(), idx, w)
    d, used = r["dispatch"], r["rows_used"]
    # expert outputs of the ledger's toy experts, raw (the combine applies w)
    y = np.zeros((used, 2), np.float32)
    rexp = row_experts(r["layout"]["expert_offsets"], used)
    for p in range(used):
        y[p] = (rexp[p] + 1) * bits_to_f32(d["recv_x"][p])
    g = np.zeros((4, 2), np.float32)
    g[0] = fx.nums("grad_out.a")
    res = oracle.combine_backward(bf16_bits_exact(g), d["tok_slot_row"], w, bf16_bits_exact(y), used)
    assert list(res["grad_w"][0]) == fx.nums("grad_w.a")
    assert np.all(res["grad_w"][1:] == 0)
    rows = d["tok_slot_row"][0]
    want = np.array(fx.nums("grad_rows.a")).reshape(2, 2)
    got = bits_to_f32(res["grad_expert_out"][rows])
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-12)
    # every other token's rows get zero gradient
    others = np.setdiff1d(np.arange(used), rows)
    assert np.all(res["grad_expert_out"][others] == 0)


class _OracleBE:
    hidden_multiple = 1

    def layout(self, idx, E, R, A):
        return oracle.layout(idx, E, R, A)

    def dispatch(self, x, idx, w, E, R, A, fp8, cap):
        return oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=cap)

    def combine(self, y, tsr, w):
        return oracle.combine(y, tsr, w)[0]


def _case(seed, A=1):
    rng = np.random.default_rng(seed)
    T, H, k, E, R = 37, 24, 3, 8, 2
    idx = random_routes(rng, T, E, k, mask_prob=0.15)
    w = rng.random((T, k)).astype(np.float32)
    x = _rand_bf16(rng, (T, H))
    d = oracle.dispatch(x, idx, w, E, R, A)
    used = int(oracle.layout(idx, E, R, A)["expert_offsets"][-1])
    return rng, T, H, k, idx, w, x, d, used


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_backward_is_the_adjoint(seed):
    """sum_p <dispatch(x)_p, G_p> == sum_t <x_t, dispatch_backward(G)_t>."""
    rng, T, H, k, idx, w, x, d, used = _case(seed)
    G = _rand_bf16(rng, (used, H))
    _, acc = oracle.dispatch_backward(G, d["tok_slot_row"])
    xf = bits_to_f32(x).astype(np.float64)
    Gf = bits_to_f32(G).astype(np.float64)
    lhs = float(sum(np.dot(xf[d["row_src"][p] // k], Gf[p]) for p in range(used)))
    rhs = float((xf * acc.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= k * 2.0 ** -24 * float(np.abs(xf).max() * np.abs(Gf).sum()) + 1e-9


@pytest.mark.parametrize("seed", range(6))
def test_combine_backward_rows_are_the_adjoint(seed):
    """sum_t <combine(y)_t, g_t> == sum_p <y_p, grad_y_p> with grad_y the
    gate times g (checked against torch's bf16 rounding of the fp32 product)."""
    rng, T, H, k, idx, w, x, d, used = _case(seed)
    y = _rand_bf16(rng, (used, H))
    g = _rand_bf16(rng, (T, H))
    _, acc = oracle.combine(y, d["tok_slot_row"], w)
    res = oracle.combine_backward(g, d["tok_slot_row"], w, y, used)
    gf = bits_to_f32(g)
    for t in range(T):
        for j in range(k):
            p = d["tok_slot_row"][t, j]
            if p < 0:
                continue
            prod = torch.from_numpy(np.float32(w[t, j]) * gf[t]).to(torch.bfloat16)
            assert np.array_equal(res["grad_expert_out"][p],
                                  prod.view(torch.int16).numpy().view(np.uint16))
    lhs = float((acc.astype(np.float64) * gf.astype(np.float64)).sum())
    yf = bits_to_f32(y).astype(np.float64)
    exact_rows = np.zeros_like(yf)
    for t in range(T):
        for j in range(k):
            p = d["tok_slot_row"][t, j]
            if p >= 0:
                exact_rows[p] = np.float64(w[t, j]) * gf[t].astype(np.float64)
    rhs = float((yf * exact_rows).sum())
    scale = float(np.abs(yf).sum() * np.abs(gf).max())
    assert abs(lhs - rhs) <= 2 * k * 2.0 ** -24 * scale + 1e-9


@pytest.mark.parametrize("seed", range(4))
def test_gate_gradient_by_finite_difference(seed):
    """F(w) = sum_{t,c} g[t,c] * combine(y; w)[t,c] is linear in each gate, so
    a central difference of the forward combine (fp32 accumulator) gives
    dF/dw[t,j] up to the fp32 rounding of the two accumulators."""
    rng, T, H, k, idx, w, x, d, used = _case(seed)
    y = _rand_bf16(rng, (used, H))
    g = _rand_bf16(rng, (T, H))
    gf = bits_to_f32(g).astype(np.float64)
    res = oracle.combine_backward(g, d["tok_slot_row"], w, y, used)
    h = np.float32(0.5)
    for t in range(0, T, 5):
        for j in range(k):
            if d["tok_slot_row"][t, j] < 0:
                assert res["grad_w"][t, j] == 0
                continue
            wp, wm = w.copy(), w.copy()
            wp[t, j] += h
            wm[t, j] -= h
            _, ap = oracle.combine(y, d["tok_slot_row"], wp)
            _, am = oracle.combine(y, d["tok_slot_row"], wm)
            fd = float(((ap[t].astype(np.float64) - am[t].astype(np.float64)) * gf[t]).sum()) / (2 * float(h))
            bound = 4 * k * 2.0 ** -24 * float(np.abs(gf[t]) @ (np.abs(ap[t]) + np.abs(am[t]))) / (2 * float(h))
            assert abs(fd - res["grad_w"][t, j]) <= bound + 1e-9


def test_gate_gradient_brute_force_tiny():
    rng = np.random.default_rng(11)
    T, H, k, cap = 4, 3, 2, 8
    tsr = np.array([[0, 5], [1, -1], [-1, -1], [7, 2]], np.int32)
    y = _rand_bf16(rng, (cap, H))
    g = _rand_bf16(rng, (T, H))
    res = oracle.combine_backward(g, tsr, None, y, cap)
    yv, gv = bits_to_f32(y).tolist(), bits_to_f32(g).tolist()
    for t in range(T):
        for j in range(k):
            p = tsr[t][j]
            want = 0.0 if p < 0 else sum(float(yv[p][c]) * float(gv[t][c]) for c in range(H))
            assert res["grad_w"][t][j] == want


@pytest.mark.parametrize("seed", range(4))
def test_transpose_duality_unweighted(seed):
    """For unweighted routes the two directions are each other's transposes:
    the backward of dispatch is combine without gates, and the row gradient
    of an ungated combine is dispatch of grad_out."""
    rng, T, H, k, idx, w, x, d, used = _case(seed, A=2)
    G = _rand_bf16(rng, (d["recv_x"].shape[0], H))
    gx, _ = oracle.dispatch_backward(G, d["tok_slot_row"])
    cx, _ = oracle.combine(G, d["tok_slot_row"], None)
    assert np.array_equal(gx, cx)
    g = _rand_bf16(rng, (T, H))
    res = oracle.combine_backward(g, d["tok_slot_row"], None, None, used, capacity=G.shape[0],
                                  fill=0x7777)
    fwd = oracle.dispatch(g, idx, None, 8, 2, 2)
    assert np.array_equal(res["grad_expert_out"][:used], fwd["recv_x"][:used])  # padding rows zero in both
