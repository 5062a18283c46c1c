"""GPU edge cases: the FP8 encoder over every bf16 value it can see at unit
scale, empty and degenerate inputs, the implementation limits, device-side
error reporting, alignment padding, rank-count independence and
determinism.  Each case is compared with the CPU oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.ep_cases import bits_to_f32  # noqa: E402
from tests.gpu_backend import GpuBackend, dev, dev_bf16, host_bf16, say  # noqa: E402

GPU = GpuBackend()


def test_fp8_encoder_every_bf16_value_at_unit_scale():
    """Blocks whose largest magnitude is 448 get scale exactly 1, so the codes
    are the E4M3 rounding of the bf16 values themselves: every finite bf16
    value with |v| <= 448 (ties, subnormal codes, signed zeros included)."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits_to_f32(allbits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    pool = allbits[keep]
    per = 127
    nblk = -(-len(pool) // per)
    blocks = np.zeros((nblk, 128), np.uint16)
    flat = np.concatenate([pool, np.zeros(nblk * per - len(pool), np.uint16)])
    blocks[:, :per] = flat.reshape(nblk, per)
    blocks[:, per] = np.where(np.arange(nblk) % 2 == 0, 0x43E0, 0xC3E0)  # +-448
    H = 1024
    T = -(-nblk // 8)
    x = np.zeros((T * 8, 128), np.uint16)
    x[:nblk] = blocks
    x[nblk:, 0] = 0x43E0
    x = x.reshape(T, H)
    idx = np.zeros((T, 1), np.int32)
    dg = GPU.dispatch(x, idx, None, 1, 1, 1, True, T)
    do = oracle.dispatch(x, idx, None, 1, 1, fp8=True, capacity=T)
    assert np.all(do["recv_scales"] == 1.0)
    assert np.array_equal(dg["recv_scales"], do["recv_scales"])
    assert np.array_equal(dg["recv_x"], do["recv_x"])


def test_fp8_zero_and_tiny_blocks():
    H = 512
    x = np.zeros((3, H), np.uint16)
    x[0, 128:256] = 0x8000                       # -0 only: amax 0 -> scale 0, codes 0
    x[1, :128] = 0x0001                          # bf16 subnormal block
    x[1, 128] = 0x8001
    x[2] = W.normal_bf16(np.random.default_rng(3), (1, H), 1e-30)
    idx = np.array([[0, 1]] * 3, np.int32)
    dg = GPU.dispatch(x, idx, None, 2, 1, 1, True, 6)
    do = oracle.dispatch(x, idx, None, 2, 1, fp8=True, capacity=6)
    assert np.array_equal(dg["recv_x"], do["recv_x"])
    assert np.array_equal(dg["recv_scales"].view(np.uint32), do["recv_scales"].view(np.uint32))


def test_empty_batch():
    E, R, k, H = 8, 2, 2, 256
    b = ep.EpBuffers(0, H, k, E, R, 1, fp8=True)
    idx = torch.zeros((0, k), dtype=torch.int32, device="cuda")
    say("empty batch")
    assert b.layout(idx, sync=True) == 0
    assert torch.all(b.expert_offsets == 0) and torch.all(b.num_tokens_per_rank == 0)
    b.dispatch(torch.zeros((0, H), dtype=torch.bfloat16, device="cuda"), idx,
               torch.zeros((0, k), dtype=torch.float32, device="cuda"))
    out = b.combine(torch.zeros((0, H), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((0, k), dtype=torch.float32, device="cuda"))
    b.check_status()
    assert out.shape == (0, H)


def test_all_masked_and_nan_gates():
    rng = np.random.default_rng(4)
    T, H, k, E, R = 70, 136, 3, 6, 3
    idx = W.random_routes(rng, T, E, k)
    idx[::3] = -1                                   # tokens with no expert at all
    idx[1::3, 1] = -1
    w = rng.random((T, k)).astype(np.float32)
    w[idx < 0] = np.nan                             # must never be read
    x = W.normal_bf16(rng, (T, H))
    dg = GPU.dispatch(x, idx, w, E, R, 1, False, T * k)
    do = oracle.dispatch(x, idx, w, E, R, 1, capacity=T * k)
    assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
    y = W.normal_bf16(rng, (T * k, H))
    og = GPU.combine(y, do["tok_slot_row"], w)
    oo, _ = oracle.combine(y, do["tok_slot_row"], w)
    assert np.array_equal(og, oo)
    assert np.all(og[::3] == 0)                     # +0, not -0, not NaN


def test_hot_expert():
    """Every token picks expert 0 (plus others): one segment holds all T
    rows, in token order."""
    rng = np.random.default_rng(5)
    T, H, k, E, R = 3000, 264, 4, 16, 4
    idx = np.concatenate([np.zeros((T, 1), np.int32),
                          1 + W.random_routes(rng, T, E - 1, k - 1)], axis=1)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    lg, lo = GPU.layout(idx, E, R, 1), oracle.layout(idx, E, R, 1)
    assert lg["num_tokens_per_expert"][0] == T
    for key in lo:
        assert np.array_equal(lg[key], lo[key])
    dg = GPU.dispatch(x, idx, w, E, R, 1, False, T * k)
    do = oracle.dispatch(x, idx, w, E, R, 1, capacity=T * k)
    assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
    assert np.array_equal(dg["recv_x"], do["recv_x"])


@pytest.mark.parametrize("case", ["max_experts", "max_topk", "max_ranks"])
def test_implementation_limits(case):
    rng = np.random.default_rng(6)
    T, H = 777, 128
    E, R, k = {"max_experts": (1024, 8, 8), "max_topk": (64, 8, 32),
               "max_ranks": (128, 64, 8)}[case]
    idx = W.random_routes(rng, T, E, k, mask_prob=0.05)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    lg, lo = GPU.layout(idx, E, R, 2), oracle.layout(idx, E, R, 2)
    for key in lo:
        assert np.array_equal(lg[key], lo[key]), key
    cap = T * k + E
    for fp8 in (False, True):
        dg = GPU.dispatch(x, idx, w, E, R, 2, fp8, cap)
        do = oracle.dispatch(x, idx, w, E, R, 2, fp8=fp8, capacity=cap)
        used = int(lo["expert_offsets"][-1])
        assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
        assert np.array_equal(dg["recv_x"][:used], do["recv_x"][:used])
        assert np.array_equal(dg["row_src"][:used], do["row_src"][:used])
    y = W.normal_bf16(rng, (cap, H))
    assert np.array_equal(GPU.combine(y, do["tok_slot_row"], w),
                          oracle.combine(y, do["tok_slot_row"], w)[0])


@pytest.mark.parametrize("H,fp8", [(65536 + 8, False), (32768, True)])
def test_wide_rows(H, fp8):
    """Rows of many chunks (64 and more per token), bf16 with a ragged
    8-column tail and FP8 with 256 scale blocks, through dispatch and
    combine."""
    T, k, E, R = 37, 4, 16, 4
    rng = np.random.default_rng(H)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.1)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    cap = T * k
    dg = GPU.dispatch(x, idx, w, E, R, 1, fp8, cap)
    do = oracle.dispatch(x, idx, w, E, R, 1, fp8=fp8, capacity=cap)
    used = int(oracle.layout(idx, E, R, 1)["expert_offsets"][-1])
    assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
    assert np.array_equal(dg["recv_x"][:used], do["recv_x"][:used])
    if fp8:
        assert np.array_equal(dg["recv_scales"][:used].view(np.uint32),
                              do["recv_scales"][:used].view(np.uint32))
    y = W.normal_bf16(rng, (cap, H))
    assert np.array_equal(GPU.combine(y, do["tok_slot_row"], w),
                          oracle.combine(y, do["tok_slot_row"], w)[0])


@pytest.mark.parametrize("T,H,mask", [(8191, 512, 0.0), (8193, 512, 0.05), (4097, 1024, 0.3),
                                      (16385, 512, 0.0), (5000, 8, 0.05)])
def test_combine_both_gather_widths(T, H, mask):
    """Combine gathers a token's rows one at a time, except in the launch's
    last 8192 work items (one wave per token and 512-column chunk), which
    gather all of them at once; a grid of at most 8192 items is all tail.
    Grids just below, at and above that size, with masked slots, weighted
    and unweighted, bit for bit against the oracle."""
    k, E, R = 8, 64, 8
    rng = np.random.default_rng(T * 7 + H)
    idx = W.random_routes(rng, T, E, k, mask_prob=mask)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    cap = T * k
    tsr = oracle.dispatch(x, idx, w, E, R, 1, fp8=False, capacity=cap)["tok_slot_row"]
    y = W.normal_bf16(rng, (cap, H))
    for weights in (w, None):
        assert np.array_equal(GPU.combine(y, tsr, weights), oracle.combine(y, tsr, weights)[0])


def _raw_run(T, H, k, E, R, idx, capacity=None, x=None):
    b = ep.EpBuffers(T, H, k, E, R, 1, capacity=capacity)
    b.status.zero_()
    idx_d = dev(idx)
    b.layout(idx_d)
    xs = dev_bf16(np.zeros((T, H), np.uint16) if x is None else x)
    b.dispatch(xs, idx_d, None)
    return b


def test_invalid_routes_reported():
    T, H, k, E, R = 40, 64, 2, 8, 2
    for bad in ("duplicate", "too_large", "below_minus_one"):
        say(f"invalid route: {bad}")
        idx = np.tile(np.array([[0, 1]], np.int32), (T, 1))
        if bad == "duplicate":
            idx[7] = [3, 3]
        elif bad == "too_large":
            idx[9, 1] = E
        else:
            idx[11, 0] = -5
        b = _raw_run(T, H, k, E, R, idx)
        with pytest.raises(ep.EpError) as e:
            b.check_status()
        assert e.value.status == ep.EP_ERR_INVALID_ROUTE


def test_capacity_too_small_reported_and_bounded():
    T, H, k, E, R = 50, 64, 2, 4, 2
    idx = np.tile(np.array([[0, 3]], np.int32), (T, 1))
    x = W.normal_bf16(np.random.default_rng(7), (T, H))
    say("capacity too small")
    b = _raw_run(T, H, k, E, R, idx, capacity=60, x=x)
    with pytest.raises(ep.EpError) as e:
        b.check_status()
    assert e.value.status == ep.EP_ERR_CAPACITY
    tsr = b.tok_slot_row.cpu().numpy()
    assert tsr.max() < 60
    # the rows that fit are still right
    do = oracle.dispatch(x, idx, None, E, R, capacity=T * k)
    fit = do["tok_slot_row"] < 60
    assert np.array_equal(tsr[fit], do["tok_slot_row"][fit])
    assert np.all(tsr[~fit] == -1)


def test_workspace_from_other_config_rejected():
    T, H, k, E, R = 64, 64, 2, 8, 2
    idx = np.tile(np.array([[0, 5]], np.int32), (T, 1))
    b = ep.EpBuffers(T, H, k, E, R, 1)
    b.status.zero_()
    b.layout(dev(idx))
    say("workspace mismatch")
    other = ep.ep_config_t(T // 2, H, k, E, R, 1)
    ep.ep_dispatch(other, ep.EP_DTYPE_BF16, dev_bf16(np.zeros((T // 2, H), np.uint16)),
                   dev(idx[: T // 2]), None, b.expert_offsets, b.workspace, b.capacity,
                   b.recv_x, None, None, b.tok_slot_row[: T // 2].contiguous(), b.row_src,
                   b.status)
    with pytest.raises(ep.EpError) as e:
        b.check_status()
    assert e.value.status == ep.EP_ERR_WORKSPACE


def test_rank_count_moves_partitions_not_rows():
    """Same routes on R = 1, 2, 8 logical ranks: expert-major rows are
    identical, rank partitions and distinct-token counts change."""
    rng = np.random.default_rng(8)
    T, H, k, E = 500, 256, 4, 32
    idx = W.random_routes(rng, T, E, k)
    x = W.normal_bf16(rng, (T, H))
    base = None
    for R in (1, 2, 8):
        d = GPU.dispatch(x, idx, None, E, R, 1, False, T * k)
        lay = GPU.layout(idx, E, R, 1)
        lo = oracle.layout(idx, E, R, 1)
        assert np.array_equal(lay["rank_offsets"], lo["rank_offsets"])
        assert np.array_equal(lay["num_tokens_per_rank"], lo["num_tokens_per_rank"])
        if base is None:
            base = d["recv_x"]
        assert np.array_equal(d["recv_x"], base)


def test_deterministic_repeat():
    w = W.WORKLOADS["skewed"]
    inp = W.generate(w)
    outs = []
    for rep in range(2):
        say(f"determinism repeat {rep}")
        b = ep.EpBuffers(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks)
        idx, wts = dev(inp["topk_idx"]), dev(inp["topk_weights"])
        b.layout(idx)
        b.dispatch(dev_bf16(inp["x"]), idx, wts)
        out = b.combine(dev_bf16(inp["y"]), wts)
        b.check_status()
        used = int(b.expert_offsets[-1].item())
        outs.append((host_bf16(b.recv_x[:used]), b.row_src[:used].cpu().numpy(),
                     b.tok_slot_row.cpu().numpy(), host_bf16(out)))
    for a, c in zip(*outs):
        assert np.array_equal(a, c)


def test_identity_round_trip_gpu():
    """bf16 dispatch, identity experts, combine with gates summing to one:
    the input comes back (as values)."""
    w = W.WORKLOADS["decode"]
    inp = W.generate(w, with_y=False)
    idx = inp["topk_idx"]
    g64 = inp["topk_weights"].astype(np.float64)
    g = (g64 / g64.sum(axis=1, keepdims=True)).astype(np.float32)
    b = ep.EpBuffers(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks)
    idx_d, g_d = dev(idx), dev(g)
    b.layout(idx_d)
    b.dispatch(dev_bf16(inp["x"]), idx_d, g_d)
    out = b.combine(b.recv_x, g_d)
    b.check_status()
    assert np.array_equal(bits_to_f32(host_bf16(out)), bits_to_f32(inp["x"]))


def test_workspace_reused_across_layouts():
    """One workspace, several layouts with different routes in a row: each
    layout's last workgroup resets the ticket for the next one."""
    rng = np.random.default_rng(9)
    T, H, k, E, R = 1500, 128, 6, 48, 4
    b = ep.EpBuffers(T, H, k, E, R, 1)
    for rep in range(5):
        say(f"workspace reuse {rep}")
        idx = W.random_routes(rng, T, E, k, mask_prob=0.1 * rep)
        x = W.normal_bf16(rng, (T, H))
        b.status.zero_()
        idx_d = dev(idx)
        rows = b.layout(idx_d, sync=True)
        b.dispatch(dev_bf16(x), idx_d, None)
        b.check_status()
        lo = oracle.layout(idx, E, R, 1)
        do = oracle.dispatch(x, idx, None, E, R, capacity=T * k)
        assert rows == lo["expert_offsets"][-1]
        assert np.array_equal(b.expert_offsets.cpu().numpy(), lo["expert_offsets"])
        assert np.array_equal(b.num_tokens_per_rank.cpu().numpy(), lo["num_tokens_per_rank"])
        assert np.array_equal(b.tok_slot_row.cpu().numpy(), do["tok_slot_row"])
        assert np.array_equal(host_bf16(b.recv_x[:rows]), do["recv_x"][:rows])


@pytest.mark.parametrize("T,E,k", [(255, 16, 3), (256, 16, 3), (257, 16, 3), (1, 256, 8),
                                   (2049, 256, 8), (1537, 512, 8), (1000, 1024, 4),
                                   (5000, 1024, 4), (4096, 64, 4), (4096, 256, 8),
                                   (4097, 256, 8), (6145, 256, 8), (8192, 256, 8),
                                   (8193, 64, 6), (9000, 128, 12), (16384, 256, 8),
                                   (16385, 256, 8), (18433, 256, 8), (16384, 64, 20),
                                   (16385, 32, 2), (70001, 32, 2), (3000, 6, 2), (5000, 6, 2),
                                   (5000, 250, 5)])
def test_layout_tile_boundaries(T, E, k):
    """Layout counts 256-token tiles in separate workgroups (one workgroup
    skips the ticket); ranks must carry across tile boundaries.  The
    scanning workgroup reads the tile rows back per expert column up to 16
    tiles of at most 256 experts, else by column quads in slices of tiles
    held in registers (up to 8 or 24 per thread) or read twice (longer
    slices, or more than 1024 columns).  The cases sit on each side of
    those limits (16/17 tiles, 24/25 tiles per slice, 64/65/73 tiles), take
    expert and rank counts that are not multiples of 4 (padded rows), and k
    in each of the kernel's register bounds (8, 16, 32)."""
    rng = np.random.default_rng(T + E)
    R = 8 if E % 8 == 0 else 1
    idx = W.random_routes(rng, T, E, k, mask_prob=0.03)
    lg, lo = GPU.layout(idx, E, R, 1), oracle.layout(idx, E, R, 1)
    for key in lo:
        assert np.array_equal(lg[key], lo[key]), key
    x = W.normal_bf16(rng, (T, 8))
    dg = GPU.dispatch(x, idx, None, E, R, 1, False, T * k)
    do = oracle.dispatch(x, idx, None, E, R, capacity=T * k)
    assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
    used = int(lo["expert_offsets"][-1])
    assert np.array_equal(dg["row_src"][:used], do["row_src"][:used])


@pytest.mark.parametrize("T,E,k", [(4096, 256, 8), (6000, 256, 8), (20000, 64, 6)])
def test_layout_outputs_at_unaligned_addresses(T, E, k):
    """The layout writes a token's rank mask, and the scan its per-expert
    counts and offsets, with 8- or 16-byte stores where the caller's arrays
    are aligned for them.  Arrays that start one element (one byte for the
    mask) past an aligned address must get the same values, by the narrow
    stores."""
    rng = np.random.default_rng(T + E + 5)
    R = 8
    idx = W.random_routes(rng, T, E, k, mask_prob=0.05)
    lo = oracle.layout(idx, E, R, 1)
    cfg = ep.ep_config_t(T, 8, k, E, R, 1)
    i32 = dict(dtype=torch.int32, device="cuda")
    ntpr = torch.full((R + 1,), -3, **i32)[1:]
    ntpe = torch.full((E + 1,), -3, **i32)[1:]
    eoff = torch.full((E + 2,), -3, **i32)[1:]
    roff = torch.full((R + 2,), -3, **i32)[1:]
    itir = torch.full((T * R + 1,), 7, dtype=torch.uint8, device="cuda")[1:].view(T, R)
    ws = torch.empty(ep.ep_layout_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, **i32)
    ep.ep_workspace_init(ws)
    say(f"unaligned layout outputs T={T} E={E} k={k}")
    ep.ep_get_dispatch_layout(cfg, dev(idx), ntpr, ntpe, itir, eoff, roff, ws, status, sync=True)
    for key, got in (("num_tokens_per_rank", ntpr), ("num_tokens_per_expert", ntpe),
                     ("expert_offsets", eoff), ("rank_offsets", roff),
                     ("is_token_in_rank", itir)):
        assert np.array_equal(got.cpu().numpy(), lo[key]), key


def test_cached_route_replay():
    """One layout, several dispatches of new hidden states over the same route
    (and both payload types), each combined through its handle: the layout's
    workspace is the cached route ("Deep Dive - DeepEP", "EPHandle")."""
    rng = np.random.default_rng(21)
    T, H, k, E, R = 900, 256, 4, 32, 4
    idx = W.random_routes(rng, T, E, k, mask_prob=0.1)
    w = rng.random((T, k)).astype(np.float32)
    b16 = ep.EpBuffers(T, H, k, E, R, 1)
    idx_d, w_d = dev(idx), dev(w)
    b16.layout(idx_d)
    b8 = ep.EpBuffers(T, H, k, E, R, 1, fp8=True)
    b8.workspace = b16.workspace  # same route, same workspace
    b8.expert_offsets = b16.expert_offsets
    for rep in range(3):
        say(f"replay {rep}")
        x = W.normal_bf16(rng, (T, H), 1.0 + rep)
        b16.dispatch(dev_bf16(x), idx_d, w_d)
        b8.dispatch(dev_bf16(x), idx_d, w_d)
        y = W.normal_bf16(rng, (T * k, H))
        out = b16.combine(dev_bf16(y), w_d)
        b16.check_status()
        d16 = oracle.dispatch(x, idx, w, E, R)
        d8 = oracle.dispatch(x, idx, w, E, R, fp8=True)
        used = int(b16.expert_offsets[-1].item())
        assert np.array_equal(host_bf16(b16.recv_x[:used]), d16["recv_x"][:used])
        assert np.array_equal(b8.recv_x[:used].cpu().numpy(), d8["recv_x"][:used])
        assert np.array_equal(b8.recv_scales[:used].cpu().numpy(), d8["recv_scales"][:used])
        ref, _ = oracle.combine(y, d16["tok_slot_row"], w)
        assert np.array_equal(host_bf16(out), ref)


def test_no_sync_valid_ranges():
    """Without reading counts back: the receive buffer is sized for the worst
    case, and the device-side offsets and counts tell the caller which rows
    are data ([off[e], off[e] + cnt[e])) and which are zero padding
    ("Deep Dive - DeepEP", "Dispatch: layout, move, and epilogue")."""
    rng = np.random.default_rng(22)
    T, H, k, E, R, A = 700, 128, 3, 24, 4, 8
    idx = W.random_routes(rng, T, E, k, mask_prob=0.2)
    x = W.normal_bf16(rng, (T, H))
    b = ep.EpBuffers(T, H, k, E, R, A)
    b.recv_x.fill_(3.0)
    b.row_src.fill_(-7)
    idx_d = dev(idx)
    b.layout(idx_d)               # no sync
    b.dispatch(dev_bf16(x), idx_d, None)
    b.check_status()
    off = b.expert_offsets.cpu().numpy()
    cnt = b.num_tokens_per_expert.cpu().numpy()
    rs = b.row_src.cpu().numpy()
    rx = host_bf16(b.recv_x)
    for e in range(E):
        data = np.arange(off[e], off[e] + cnt[e])
        pad = np.arange(off[e] + cnt[e], off[e + 1])
        assert np.all(rs[data] >= 0) and np.all(idx.reshape(-1)[rs[data]] == e)
        assert np.all(rs[pad] == -1) and np.all(rx[pad] == 0)
    assert off[-1] <= b.capacity
    assert np.all(rs[off[-1]:] == -7)  # past the last segment nothing is written


def test_layout_scan_hand_off_repeated():
    """The scanning workgroup reads the other workgroups' tile counts after
    a release-acquire ticket.  Forty layouts of fresh routes over 64 tiles,
    with no synchronisation between launch and dispatch, must each match
    the oracle bit for bit (counts, offsets, rank partitions, positions)."""
    rng = np.random.default_rng(77)
    T, H, k, E, R = 16384, 8, 8, 256, 8
    b = ep.EpBuffers(T, H, k, E, R, 1)
    x = W.normal_bf16(rng, (T, H))
    x_d = dev_bf16(x)
    for rep in range(40):
        idx = W.random_routes(rng, T, E, k, mask_prob=0.02 * (rep % 3))
        idx_d = dev(idx)
        b.layout(idx_d)
        b.dispatch(x_d, idx_d, None)
        torch.cuda.synchronize()
        b.check_status()
        lo = oracle.layout(idx, E, R, 1)
        do = oracle.dispatch(x, idx, None, E, R, capacity=T * k)
        for key in ("num_tokens_per_expert", "num_tokens_per_rank", "expert_offsets",
                    "rank_offsets"):
            assert np.array_equal(getattr(b, key).cpu().numpy(), lo[key]), (rep, key)
        assert np.array_equal(b.tok_slot_row.cpu().numpy(), do["tok_slot_row"]), rep
