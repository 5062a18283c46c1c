"""The allocation-free entry point ep_layout_dispatch_noalloc, called
through the C ABI, against the calls it stands for: ep_layout_dispatch for a
batch of at most one tile, ep_get_dispatch_layout then ep_dispatch for a
larger one.  Every output must be bit-identical, also on consecutive calls
of different sizes (the library's scratch keeps the previous call's
contents), and must match the CPU oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, dev_bf16, host_bf16, say  # noqa: E402

OUTS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "expert_offsets",
        "rank_offsets", "tok_slot_row")


def _case(seed, T, H, k, E, R, A, fp8):
    rng = np.random.default_rng(seed)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.05)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    return idx, x, w


def _noalloc(b, x, idx, w):
    return ep.ep_layout_dispatch_noalloc(
        b.cfg, ep.EP_DTYPE_FP8_E4M3 if b.fp8 else ep.EP_DTYPE_BF16, x, idx, w,
        b.num_tokens_per_rank, b.num_tokens_per_expert, b.is_token_in_rank, b.expert_offsets,
        b.rank_offsets, b.capacity, b.recv_x, b.recv_scales, b.recv_weights, b.tok_slot_row,
        b.row_src, b.status)


def _host(b, rows):
    got = {n: getattr(b, n).cpu().numpy() for n in OUTS}
    got["recv_x"] = b.recv_x[:rows].cpu().numpy() if b.fp8 else host_bf16(b.recv_x[:rows])
    if b.fp8:
        got["recv_scales"] = b.recv_scales[:rows].cpu().numpy().view(np.uint32)
    got["recv_weights"] = b.recv_weights[:rows].cpu().numpy().view(np.uint32)
    got["row_src"] = b.row_src[:rows].cpu().numpy()
    return got


def _check_case(name, seed, T, H, k, E, R, A, fp8):
    idx, x, w = _case(seed, T, H, k, E, R, A, fp8)
    say(f"noalloc {name}: T={T} H={H} k={k} E={E} R={R} A={A} fp8={fp8}")
    idx_d, x_d, w_d = dev(idx), dev_bf16(x), dev(w)
    ref = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    ref.layout_and_dispatch(x_d, idx_d, w_d)
    ref.check_status()
    na = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    h = _noalloc(na, x_d, idx_d, w_d)
    na.check_status()
    rows = int(ref.expert_offsets[-1].item())
    a, b = _host(ref, rows), _host(na, rows)
    for key in a:
        assert np.array_equal(a[key], b[key]), f"{name}: {key} differs from the two-call path"
    # and the oracle
    lay = oracle.layout(idx, E, R, A)
    do = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=na.capacity)
    for key in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
                "expert_offsets", "rank_offsets"):
        assert np.array_equal(b[key], lay[key]), f"{name}: {key} differs from the oracle"
    assert np.array_equal(b["tok_slot_row"], do["tok_slot_row"])
    assert np.array_equal(b["recv_x"], do["recv_x"][:rows])
    assert np.array_equal(b["row_src"], do["row_src"][:rows])
    if fp8:
        assert np.array_equal(b["recv_scales"], do["recv_scales"][:rows].view(np.uint32))
    # combine through the returned handle
    y = W.normal_bf16(np.random.default_rng(seed + 1), (na.capacity, H))
    y_d = dev_bf16(y)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(h, y_d, w_d, out)
    ref_out, _ = oracle.combine(y, do["tok_slot_row"], w)
    assert np.array_equal(host_bf16(out), ref_out)


def test_noalloc_matches_the_calls_it_stands_for_on_consecutive_calls():
    # larger first, then smaller ones: the scratch keeps the last call's contents
    _check_case("prefill", 3, 4096, 7168, 8, 256, 8, 1, True)
    _check_case("multi-tile bf16", 4, 1000, 1024, 6, 64, 8, 4, False)
    _check_case("one tile", 5, 200, 2048, 6, 64, 8, 4, False)
    _check_case("one tile fp8", 6, 96, 512, 4, 16, 4, 1, True)


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    T, k, E, R = 200000, 8, 256, 8
    cfg = ep.ep_config_t(T, 128, k, E, R, 1)
    assert ep.ep_layout_workspace_bytes(cfg) > ep.NOALLOC_SCRATCH_BYTES
    P = torch.empty(16, dtype=torch.uint8, device="cuda")
    import ctypes

    st = ep.lib().ep_layout_dispatch_noalloc(
        ctypes.byref(cfg), ep.EP_DTYPE_BF16, *([ctypes.c_void_p(P.data_ptr())] * 8), T * k, 1,
        *([ctypes.c_void_p(P.data_ptr())] * 6), None, None)
    assert st == ep.EP_ERR_INVALID_ARG
    assert b"scratch" in ep.lib().ep_last_error_string()
