"""Randomized parity sweep, bounded and reproducible: shapes drawn from
fixed seeds, each run through every path the library offers and compared
with the CPU oracle bit for bit (combine as bf16 bits, gate gradients
within their fp32 bound):

- layout (every output), dispatch (handle, rows, scales, gates) and
  combine through the two-call path;
- ep_layout_dispatch against the two-call path, workspace included;
- the non-expanded path (dispatch_ranked, expand, ranked combine);
- both backward calls (bf16 rows).

Half the shapes are general (T up to 20000, H up to 1592, k up to 32, E up
to 256, R up to 64, A up to 16, masks up to 30%, both payload types); the
other half sit at the layout's tile and read-back boundaries (255-257,
4095-4097, 8191-8193, 16383-16385 tokens) or have up to 1024 experts, so
that scanning threads own several experts.  Each case prints its shape
before it runs, and -x stops the run at the first mismatch.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests import test_gpu_backward as TB  # noqa: E402
from tests import test_gpu_layout_dispatch as TL  # noqa: E402
from tests import test_gpu_ranked as TR  # noqa: E402
from tests.gpu_backend import GpuBackend, say  # noqa: E402

GPU = GpuBackend()
N_GENERAL, N_EDGE = 24, 24


def _draw(rng, edges):
    R = int(rng.choice([1, 2, 4, 8, 16, 64]))
    E = min(R * int(rng.integers(1, max(2, (1024 if edges else 256) // R + 1))), 1024)
    k = int(rng.integers(1, min(E, 32) + 1))
    fp8 = bool(rng.integers(0, 2))
    H = 128 * int(rng.integers(1, 13)) if fp8 else 8 * int(rng.integers(1, 200))
    if edges:
        T = int(rng.choice([255, 256, 257, 4095, 4096, 4097, 8191, 8192, 8193, 16383, 16384,
                            16385, int(rng.integers(1, 20000))]))
    else:
        T = int(rng.choice([int(rng.integers(0, 300)), int(rng.integers(0, 3000)),
                            int(rng.integers(3000, 20000))]))
    if T > 3000:  # keeps the oracle's share of the run to seconds
        H = 128 * int(rng.integers(1, 3)) if fp8 else 8 * int(rng.integers(1, 33))
    A = int(rng.choice([1, 1, 2, 4, 16]))
    mask = float(rng.choice([0.0, 0.05, 0.3]))
    return T, H, k, E, R, A, fp8, mask, int(rng.integers(0, 1 << 30))


def _cases():
    general = np.random.default_rng(9000)
    edge = np.random.default_rng(9100)
    return ([("general", i, _draw(general, False)) for i in range(N_GENERAL)]
            + [("edge", i, _draw(edge, True)) for i in range(N_EDGE)])


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}{}_T{}_H{}_k{}_E{}_R{}_A{}".format(
    c[0], c[1], *c[2][:6]))
def test_random_shape_through_every_path(case):
    T, H, k, E, R, A, fp8, mask, seed = case[2]
    say(f"sweep {case[0]} {case[1]}: T={T} H={H} k={k} E={E} R={R} A={A} fp8={fp8} "
        f"mask={mask} seed={seed}")
    rng = np.random.default_rng(seed)
    idx = W.random_routes(rng, T, E, k, mask_prob=mask) if T else np.zeros((0, k), np.int32)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    cap = T * k + E * (A - 1)
    y = W.normal_bf16(rng, (cap, H))
    TL._check_against_two_calls(T, H, k, E, R, A, fp8, bool(seed & 1), seed=seed)
    if T == 0:
        return
    lg, lo = GPU.layout(idx, E, R, A), oracle.layout(idx, E, R, A)
    for key in lo:
        assert np.array_equal(lg[key], lo[key]), key
    dg = GPU.dispatch(x, idx, w, E, R, A, fp8, cap)
    do = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=cap)
    used = int(lo["expert_offsets"][-1])
    assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
    for key in ("row_src", "recv_x", "recv_weights") + (("recv_scales",) if fp8 else ()):
        assert np.array_equal(dg[key][:used], do[key][:used]), key
    assert np.array_equal(GPU.combine(y, do["tok_slot_row"], w),
                          oracle.combine(y, do["tok_slot_row"], w)[0])
    TR.check(T, H, k, E, R, A, fp8, idx, w, x, y, weighted=bool(seed & 2))
    if not fp8:
        g = W.normal_bf16(rng, (T, H))
        TB.check_against_oracle(T, H, k, E, R, A, idx, w, x, y, g, weighted=bool(seed & 4),
                                want_gate=bool(seed & 8))
