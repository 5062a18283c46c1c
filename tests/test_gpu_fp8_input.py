"""GPU parity of ep_dispatch_fp8_input (pre-quantised rows) against the
oracle: codes, scales, handle and gates bit-exact, at the Prefill and Large
shapes and on ragged small shapes with alignment padding."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, say  # noqa: E402


def run(T, H, k, E, R, A, idx, w, codes, scales):
    say(f"fp8 input T={T} H={H} k={k} E={E} R={R} A={A}")
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=True)
    b.row_src.fill_(-2)
    idx_d = dev(idx)
    rows = b.layout(idx_d, sync=True)
    b.dispatch_fp8_input(dev(codes), dev(scales), idx_d, dev(w))
    b.check_status()
    o = oracle.dispatch_fp8_input(codes, scales, idx, w, E, R, A)
    assert np.array_equal(b.tok_slot_row.cpu().numpy(), o["tok_slot_row"])
    for name in ("recv_x", "recv_scales", "recv_weights", "row_src"):
        got = getattr(b, name)[:rows].cpu().numpy()
        assert np.array_equal(got.view(np.uint8), o[name][:rows].view(np.uint8)), name


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["prefill", "large"])
def test_fp8_input_workloads(name):
    w = W.WORKLOADS[name]
    inp = W.generate(w, with_y=False)
    rng = np.random.default_rng(500 + w.seed)
    codes = rng.integers(0, 256, (w.num_tokens, w.hidden), dtype=np.uint8)
    scales = rng.random((w.num_tokens, w.hidden // 128)).astype(np.float32)
    run(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, 1,
        inp["topk_idx"], inp["topk_weights"], codes, scales)


@pytest.mark.parametrize("seed", range(10))
def test_fp8_input_random_small(seed):
    rng = np.random.default_rng(900 + seed)
    T = int(rng.choice([1, 63, 257, 800]))
    H = int(rng.choice([128, 384, 1152, 2048]))
    R = int(rng.choice([1, 2, 4]))
    E = R * int(rng.integers(1, 9))
    k = int(rng.integers(1, min(E, 8) + 1))
    A = int(rng.choice([1, 2, 8]))
    idx = W.random_routes(rng, T, E, k, mask_prob=0.15)
    w = rng.random((T, k)).astype(np.float32)
    codes = rng.integers(0, 256, (T, H), dtype=np.uint8)
    scales = rng.random((T, H // 128)).astype(np.float32)
    run(T, H, k, E, R, A, idx, w, codes, scales)
