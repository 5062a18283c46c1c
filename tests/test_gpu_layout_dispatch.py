"""ep_layout_dispatch (layout and dispatch in one call: one launch up to 256
tokens, the two calls' launches above) against the two-call path and the
oracle.

The fused call must leave exactly what ep_get_dispatch_layout followed by
ep_dispatch leaves: every layout output, every receive row, scale, gate
and handle entry, and the whole workspace.  Combine and the non-expanded
path then run on its results unchanged, and are checked against the oracle.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, dev_bf16, host_bf16, say  # noqa: E402

CASES = [
    # T, H, k, E, R, A, fp8, weighted
    (0, 256, 4, 32, 4, 1, False, True),      # empty batch
    (1, 128, 2, 8, 2, 1, False, True),
    (64, 128, 2, 8, 2, 1, False, True),      # the Tiny shape
    (128, 7168, 8, 256, 8, 1, False, True),  # the Decode shape
    (200, 1024, 8, 256, 8, 1, True, True),   # FP8, ragged tokens
    (256, 264, 3, 24, 4, 4, False, True),    # a full tile, alignment padding, H % 16 == 8
    (256, 512, 6, 48, 4, 2, True, False),    # FP8 without gates, padding
    (97, 256, 32, 64, 8, 1, False, True),    # k = 32
    (150, 128, 4, 1024, 64, 1, False, True), # E and R at their limits
    (257, 256, 4, 32, 4, 1, False, True),    # two tiles: two launches
    (1000, 1032, 6, 64, 8, 4, False, True),  # ragged tiles, padding, H % 16 == 8
    (4096, 7168, 8, 256, 8, 1, True, True),  # the Prefill shape
    (8193, 384, 6, 64, 8, 2, True, False),   # 33 tiles (four-batch scan), FP8, no gates
]

OUTPUTS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
           "expert_offsets", "rank_offsets", "tok_slot_row")


def _fresh(T, H, k, E, R, A, fp8):
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    b.workspace.zero_()  # section padding compares equal too
    ep.ep_workspace_init(b.workspace)
    b.row_src.fill_(-2)
    b.recv_weights.fill_(-3.0)
    b.recv_x.zero_()
    if fp8:
        b.recv_scales.fill_(-4.0)
    return b


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_H{}_k{}_E{}_R{}_A{}_{}{}".format(
    *c[:6], "fp8" if c[6] else "bf16", "" if c[7] else "_noweights"))
def test_layout_dispatch_equals_two_calls(case):
    _check_against_two_calls(*case, seed=900 + case[0] + case[3] + case[2])


@pytest.mark.parametrize("seed", range(24))
def test_layout_dispatch_random_shapes(seed):
    """Random shapes up to one tile: tokens, hidden size, experts, ranks,
    top-k, alignment, payload type and gates all drawn from the seed."""
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.choice([1, 2, 4, 8, 16]))
    E = R * int(rng.integers(1, 9))
    k = int(rng.integers(1, min(E, 8) + 1))
    fp8 = bool(rng.integers(0, 2))
    H = 128 * int(rng.integers(1, 7)) if fp8 else 8 * int(rng.integers(1, 161))
    T = int(rng.integers(0, 257))
    A = int(rng.choice([1, 2, 4]))
    _check_against_two_calls(T, H, k, E, R, A, fp8, bool(rng.integers(0, 2)), seed=seed)


def _check_against_two_calls(T, H, k, E, R, A, fp8, weighted, seed):
    say(f"layout_dispatch T={T} H={H} k={k} E={E} R={R} A={A} fp8={fp8} w={weighted}")
    rng = np.random.default_rng(seed)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.1) if T else np.zeros((0, k), np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    idx_d, x_d = dev(idx), dev_bf16(x)
    w_d = dev(w) if weighted else None

    two = _fresh(T, H, k, E, R, A, fp8)
    two.layout(idx_d)
    two.dispatch(x_d, idx_d, w_d)
    one = _fresh(T, H, k, E, R, A, fp8)
    one.layout_dispatch(x_d, idx_d, w_d)
    torch.cuda.synchronize()
    two.check_status()
    one.check_status()

    for name in OUTPUTS:
        assert torch.equal(getattr(one, name), getattr(two, name)), name
    assert torch.equal(one.workspace, two.workspace)
    used = int(two.expert_offsets[-1].item())
    assert torch.equal(one.row_src[:used], two.row_src[:used])
    assert torch.equal(one.recv_x[:used].view(torch.uint8), two.recv_x[:used].view(torch.uint8))
    if weighted:
        assert torch.equal(one.recv_weights[:used].view(torch.int32),
                           two.recv_weights[:used].view(torch.int32))
    if fp8:
        assert torch.equal(one.recv_scales[:used].view(torch.int32),
                           two.recv_scales[:used].view(torch.int32))

    # the oracle, and combine on the fused call's handle
    d = oracle.dispatch(x, idx, w if weighted else None, E, R, A, fp8=fp8)
    assert np.array_equal(one.tok_slot_row.cpu().numpy(), d["tok_slot_row"])
    got = one.recv_x[:used].cpu().numpy() if fp8 else host_bf16(one.recv_x[:used])
    assert np.array_equal(got, d["recv_x"][:used])
    if T:
        y = W.normal_bf16(rng, (one.capacity, H))
        out = one.combine(dev_bf16(y), dev(w))
        ref, _ = oracle.combine(y, d["tok_slot_row"], w)
        assert np.array_equal(host_bf16(out), ref)


def test_layout_dispatch_then_non_expanded_path():
    """The workspace the fused call leaves serves the non-expanded dispatch,
    expand and ranked combine (Decode shape, FP8 rows)."""
    T, H, k, E, R = 128, 1024, 8, 256, 8
    say("layout_dispatch then ranked")
    rng = np.random.default_rng(4321)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.05)
    w = rng.random((T, k)).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    b = ep.EpBuffers(T, H, k, E, R, 1, fp8=True)
    idx_d, w_d, x_d = dev(idx), dev(w), dev_bf16(x)
    b.layout_dispatch(x_d, idx_d, w_d)
    b.dispatch_ranked(x_d, idx_d, w_d)
    b.expand()
    y = W.normal_bf16(rng, (b.capacity, H))
    out = b.combine_ranked(dev_bf16(y))
    b.check_status()
    torch.cuda.synchronize()
    ne = oracle.dispatch_ranked(x, idx, w, E, R, fp8=True)
    rows = int(ne["rank_token_offsets"][-1])
    assert np.array_equal(b.rank_token_offsets.cpu().numpy(), ne["rank_token_offsets"])
    assert np.array_equal(b.ne_x[:rows].cpu().numpy(), ne["recv_x"][:rows])
    d = oracle.dispatch(x, idx, w, E, R, 1, fp8=True)
    ref, _, _ = oracle.combine_ranked(y, d["tok_slot_row"], ne, weighted=True)
    assert np.array_equal(host_bf16(out), ref)


def test_layout_dispatch_decode_workload():
    """The Decode workload through the fused call, against the oracle."""
    wl = W.WORKLOADS["decode"]
    inp = W.generate(wl)
    say("layout_dispatch decode workload")
    b = ep.EpBuffers(wl.num_tokens, wl.hidden, wl.num_topk, wl.num_experts, wl.num_ranks,
                     wl.alignment, fp8=wl.fp8)
    idx_d, w_d = dev(inp["topk_idx"]), dev(inp["topk_weights"])
    b.layout_dispatch(dev_bf16(inp["x"]), idx_d, w_d)
    out = b.combine(dev_bf16(inp["y"]), w_d)
    b.check_status()
    lay = oracle.layout(inp["topk_idx"], wl.num_experts, wl.num_ranks, wl.alignment)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_weights"], wl.num_experts,
                        wl.num_ranks, wl.alignment, fp8=wl.fp8)
    for key in ("num_tokens_per_expert", "num_tokens_per_rank", "expert_offsets",
                "rank_offsets", "is_token_in_rank"):
        assert np.array_equal(getattr(b, key).cpu().numpy(), lay[key]), key
    used = int(lay["expert_offsets"][-1])
    assert np.array_equal(host_bf16(b.recv_x[:used]), d["recv_x"][:used])
    ref, _ = oracle.combine(inp["y"], d["tok_slot_row"], inp["topk_weights"])
    assert np.array_equal(host_bf16(out), ref)


@pytest.mark.parametrize("T", [256, 257])
def test_layout_and_dispatch_picks_either_path(T):
    """EpBuffers.layout_and_dispatch runs one launch up to 256 tokens and the
    layout and dispatch launches above; both give the oracle's rows."""
    H, k, E, R = 256, 4, 32, 4
    say(f"layout_and_dispatch T={T}")
    rng = np.random.default_rng(T)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.05)
    w = rng.random((T, k)).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    b = ep.EpBuffers(T, H, k, E, R, 1)
    b.layout_and_dispatch(dev_bf16(x), dev(idx), dev(w))
    b.check_status()
    d = oracle.dispatch(x, idx, w, E, R, 1)
    used = int(b.expert_offsets[-1].item())
    assert np.array_equal(b.tok_slot_row.cpu().numpy(), d["tok_slot_row"])
    assert np.array_equal(host_bf16(b.recv_x[:used]), d["recv_x"][:used])
