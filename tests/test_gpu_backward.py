"""GPU parity for the backward calls against the CPU oracle.

ep_dispatch_backward: bit-exact (same fixed-order fp32 sum, one rounding).
ep_combine_backward: row gradients bit-exact; gate gradients are fp32 sums
of H products in a fixed (but different) order, checked against the exact
fp64 sum with the order-independent bound
    |got - exact| <= gamma_H * sum_c |y_c g_c|,  gamma_n = n u / (1 - n u),
u = 2^-24, plus the final fp32 rounding of the result (u * |exact|).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, dev_bf16, host_bf16, say  # noqa: E402

U = 2.0 ** -24


def gate_grad_ok(got, exact, mag, H):
    gamma = H * U / (1 - H * U)
    bound = gamma * mag + U * np.abs(exact) + 1e-30
    return np.abs(got.astype(np.float64) - exact) <= bound


def run_case(T, H, k, E, R, A, idx, w, x, y, g, weighted=True, want_gate=True):
    b = ep.EpBuffers(T, H, k, E, R, A)
    idx_d = dev(idx)
    w_d = dev(w) if weighted else None
    b.row_src.fill_(-2)
    rows = b.layout(idx_d, sync=True)
    b.dispatch(dev_bf16(x), idx_d, dev(w))
    y_d, g_d = dev_bf16(y), dev_bf16(g)
    gx = b.dispatch_backward(y_d)
    gy = torch.full((b.capacity, H), 7.0, dtype=torch.bfloat16, device="cuda")
    gw = torch.full((T, k), 9.0, dtype=torch.float32, device="cuda") if want_gate else None
    b.combine_backward(g_d, w_d, y_d if want_gate else None, gy, gw)
    b.check_status()
    torch.cuda.synchronize()
    return b, rows, host_bf16(gx), host_bf16(gy), (gw.cpu().numpy() if want_gate else None)


def check_against_oracle(T, H, k, E, R, A, idx, w, x, y, g, weighted=True, want_gate=True):
    b, rows, gx, gy, gw = run_case(T, H, k, E, R, A, idx, w, x, y, g, weighted, want_gate)
    d = oracle.dispatch(x, idx, w, E, R, A)
    tsr = d["tok_slot_row"]
    assert np.array_equal(b.tok_slot_row.cpu().numpy(), tsr)
    ogx, _ = oracle.dispatch_backward(y, tsr)
    assert np.array_equal(gx, ogx)
    res = oracle.combine_backward(g, tsr, w if weighted else None, y if want_gate else None, rows,
                                  capacity=y.shape[0])
    assert np.array_equal(gy[:rows], res["grad_expert_out"][:rows])
    if want_gate:
        ok = gate_grad_ok(gw, res["grad_w"], res["grad_w_abs"], H)
        assert ok.all(), f"{(~ok).sum()} gate gradients outside the bound"
    return gw


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "large"])
def test_backward_workloads(name):
    w = W.WORKLOADS[name]
    say(f"backward {name}")
    inp = W.generate(w)
    rng = np.random.default_rng(100 + w.seed)
    g = W.normal_bf16(rng, (w.num_tokens, w.hidden))
    check_against_oracle(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                         w.alignment, inp["topk_idx"], inp["topk_weights"], inp["x"], inp["y"], g)


@pytest.mark.parametrize("seed", range(16))
def test_backward_random_small(seed):
    rng = np.random.default_rng(3000 + seed)
    T = int(rng.choice([1, 7, 64, 300, 1000]))
    H = int(rng.choice([8, 24, 520, 1032, 2056]))
    R = int(rng.choice([1, 2, 4]))
    E = R * int(rng.integers(1, 9))
    k = int(rng.integers(1, min(E, 9) + 1))
    A = int(rng.choice([1, 1, 2, 4]))
    idx = W.random_routes(rng, T, E, k, mask_prob=float(rng.choice([0.0, 0.2])))
    w = rng.random((T, k)).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    cap = T * k + E * (A - 1)
    y = W.normal_bf16(rng, (cap, H))
    g = W.normal_bf16(rng, (T, H), float(rng.choice([1.0, 1e-3, 50.0])))
    check_against_oracle(T, H, k, E, R, A, idx, w, x, y, g, weighted=bool(seed % 3),
                         want_gate=bool(seed % 4 != 1))


def test_backward_deterministic():
    w = W.WORKLOADS["skewed"]
    inp = W.generate(w)
    g = W.normal_bf16(np.random.default_rng(7), (w.num_tokens, w.hidden))
    outs = [run_case(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, 1,
                     inp["topk_idx"], inp["topk_weights"], inp["x"], inp["y"], g)
            for _ in range(2)]
    rows = outs[0][1]
    assert np.array_equal(outs[0][2], outs[1][2])
    assert np.array_equal(outs[0][3][:rows], outs[1][3][:rows])
    assert np.array_equal(outs[0][4].view(np.uint32), outs[1][4].view(np.uint32))
