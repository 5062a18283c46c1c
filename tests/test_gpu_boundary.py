"""GPU checks of the boundary's failure and option contracts, each against
the CPU oracle:

- an inf or NaN among the hidden values, or in the gate of a used
  selection, sets the non-finite status bit on every dispatch path, and the
  rows of every other token stay exact ("Deep Dive - DeepEP", "A runnable
  routing ledger": such inputs are rejected; "Combine: reverse routing plus
  reduction": failure belongs at the contract boundary);
- zero_padding on and off ("Deep Dive - DeepEP", "Dispatch: layout, move,
  and epilogue": clearing alignment gaps is the caller's choice): with it
  off, padding rows keep their payload and scales but still get source -1
  and gate 0;
- a workspace that holds no layout of this configuration, or holds garbage
  counts, never makes the padding fill write outside the receive rows.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.gpu_backend import dev, dev_bf16, host_bf16, say  # noqa: E402

SENTINEL = 0x5A


def _status_of(b):
    try:
        b.check_status()
    except ep.EpError as e:
        return e.status
    return ep.EP_OK


def _rows(b, fp8):
    return b.recv_x.cpu().numpy() if fp8 else host_bf16(b.recv_x)


def _case(seed, T, H, k, E, R):
    rng = np.random.default_rng(seed)
    idx = W.random_routes(rng, T, E, k, mask_prob=0.1)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    return idx, x, w


# --------------------------------------------------------------------------
# non-finite inputs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("bad", [0x7F80, 0xFF80, 0x7FC1])  # +inf, -inf, NaN
def test_nonfinite_hidden_value_is_reported(fp8, fused, bad):
    T, H, k, E, R = 200, 512, 4, 16, 4
    idx, x, w = _case(40, T, H, k, E, R)
    tb, cb = 7, 130                                   # token 7, block 1
    xbad = x.copy()
    xbad[tb, cb] = bad
    say(f"nonfinite x fp8={fp8} fused={fused} bits={bad:#x}")
    b = ep.EpBuffers(T, H, k, E, R, 1, fp8=fp8)
    idx_d = dev(idx)
    if fused:
        b.layout_dispatch(dev_bf16(xbad), idx_d, dev(w))
    else:
        b.layout(idx_d)
        b.dispatch(dev_bf16(xbad), idx_d, dev(w))
    assert _status_of(b) == ep.EP_ERR_NONFINITE
    # every row of every other token is what the oracle gives for finite x
    do = oracle.dispatch(x, idx, w, E, R, fp8=fp8, capacity=T * k)
    tsr = b.tok_slot_row.cpu().numpy()
    assert np.array_equal(tsr, do["tok_slot_row"])
    rows = _rows(b, fp8)
    other = [p for t in range(T) if t != tb for p in tsr[t] if p >= 0]
    assert np.array_equal(rows[other], do["recv_x"][other])
    if fp8:
        got_s = b.recv_scales.cpu().numpy()
        assert np.array_equal(got_s[other].view(np.uint32), do["recv_scales"][other].view(np.uint32))
        # blocks of token 7 other than the bad one are exact too
        mine = [p for p in tsr[tb] if p >= 0]
        for blk in (0, 2, 3):
            sl = slice(128 * blk, 128 * (blk + 1))
            assert np.array_equal(rows[mine][:, sl], do["recv_x"][mine][:, sl])
    else:
        mine = [p for p in tsr[tb] if p >= 0]
        assert np.all(rows[mine][:, cb] == bad)       # the bits travel unchanged


def test_nonfinite_gate_of_a_used_selection_is_reported():
    T, H, k, E, R = 300, 256, 4, 16, 4
    idx, x, w = _case(41, T, H, k, E, R)
    t, j = np.argwhere(idx >= 0)[5]
    wbad = w.copy()
    wbad[t, j] = np.inf
    wbad[idx < 0] = np.nan                            # unused slots: never read
    say("nonfinite gate")
    b = ep.EpBuffers(T, H, k, E, R, 1)
    b.layout(dev(idx))
    b.dispatch(dev_bf16(x), dev(idx), dev(wbad))
    assert _status_of(b) == ep.EP_ERR_NONFINITE
    w_ok = w.copy()
    w_ok[idx < 0] = np.nan
    do = oracle.dispatch(x, idx, w_ok, E, R, capacity=T * k)
    M = int((idx >= 0).sum())                         # rows used (A = 1)
    assert np.array_equal(_rows(b, False)[:M], do["recv_x"][:M])
    assert np.array_equal(b.row_src.cpu().numpy()[:M], do["row_src"][:M])
    got_w = b.recv_weights.cpu().numpy()[:M]
    p_bad = do["tok_slot_row"][t, j]
    keep = np.arange(M) != p_bad
    assert np.array_equal(got_w[keep], do["recv_weights"][:M][keep]) and np.isinf(got_w[p_bad])
    # NaN only in unused slots is not an error
    b2 = ep.EpBuffers(T, H, k, E, R, 1)
    b2.layout(dev(idx))
    b2.dispatch(dev_bf16(x), dev(idx), dev(w_ok))
    assert _status_of(b2) == ep.EP_OK


@pytest.mark.parametrize("fp8", [False, True])
def test_nonfinite_on_the_non_expanded_path(fp8):
    T, H, k, E, R = 150, 384, 3, 12, 4
    idx, x, w = _case(42, T, H, k, E, R)
    xbad = x.copy()
    xbad[33, 200] = 0x7FC0
    say(f"nonfinite ranked fp8={fp8}")
    b = ep.EpBuffers(T, H, k, E, R, 1, fp8=fp8)
    b.layout(dev(idx))
    b.dispatch_ranked(dev_bf16(xbad), dev(idx), dev(w))
    assert _status_of(b) == ep.EP_ERR_NONFINITE
    ne = oracle.dispatch_ranked(x, idx, w, E, R, fp8=fp8)
    trr = b.tok_rank_row.cpu().numpy()
    assert np.array_equal(trr, ne["tok_rank_row"])
    got = b.ne_x.cpu().numpy() if fp8 else host_bf16(b.ne_x)
    other = [q for t in range(T) if t != 33 for q in trr[t] if q >= 0]
    assert np.array_equal(got[other], ne["recv_x"][other])
    # a bad gate of a used selection, on a finite row
    wbad = w.copy()
    t, j = np.argwhere(idx >= 0)[3]
    wbad[t, j] = np.nan
    b2 = ep.EpBuffers(T, H, k, E, R, 1, fp8=fp8)
    b2.layout(dev(idx))
    b2.dispatch_ranked(dev_bf16(x), dev(idx), dev(wbad))
    assert _status_of(b2) == ep.EP_ERR_NONFINITE


# --------------------------------------------------------------------------
# zero_padding
# --------------------------------------------------------------------------

def _sentinel_buffers(b, fp8):
    if fp8:
        b.recv_x.fill_(SENTINEL)
        b.recv_scales.view(torch.int32).fill_(0x5A5A5A5A)
    else:
        b.recv_x.view(torch.int16).fill_(0x5A5A)
    b.recv_weights.fill_(7.0)
    b.row_src.fill_(-2)


def _check_padding(b, do, fp8, zero_padding, rows_used, cnt, offs):
    rows = _rows(b, fp8)
    pad = np.zeros(rows_used, bool)
    for e in range(len(cnt)):
        pad[offs[e] + cnt[e]:offs[e + 1]] = True
    valid = ~pad
    assert np.array_equal(rows[:rows_used][valid], do["recv_x"][:rows_used][valid])
    assert np.all(b.row_src.cpu().numpy()[:rows_used][pad] == -1)
    assert np.all(b.recv_weights.cpu().numpy()[:rows_used][pad] == 0.0)
    if zero_padding:
        assert np.all(rows[:rows_used][pad] == 0)
        if fp8:
            assert np.all(b.recv_scales.cpu().numpy()[:rows_used][pad] == 0.0)
    else:
        want = SENTINEL if fp8 else 0x5A5A
        assert np.all(rows[:rows_used][pad] == want)
        if fp8:
            assert np.all(b.recv_scales.cpu().numpy()[:rows_used][pad].view(np.uint32)
                          == 0x5A5A5A5A)
    # rows past the used ones are never written
    assert np.all(b.row_src.cpu().numpy()[rows_used:] == -2)


@pytest.mark.parametrize("zero_padding", [True, False])
@pytest.mark.parametrize("path", ["dispatch", "fused", "fp8_input", "expand"])
@pytest.mark.parametrize("shape", ["alignment_example", "random_a16"])
def test_zero_padding_choice(zero_padding, path, shape):
    if shape == "alignment_example":
        # the page's example: counts [3, 1] with alignment 4 give starts [0, 4]
        idx = np.array([[0], [0], [0], [1]], np.int32)
        T, H, k, E, R, A = 4, 256, 1, 2, 1, 4
        x = W.normal_bf16(np.random.default_rng(43), (T, H))
        w = np.full((T, k), 0.5, np.float32)
    else:
        T, H, k, E, R, A = 180, 384, 3, 12, 4, 16
        idx, x, w = _case(44, T, H, k, E, R)
    fp8 = path in ("fp8_input",) or (path != "fused" and shape == "random_a16")
    say(f"zero_padding={zero_padding} path={path} shape={shape} fp8={fp8}")
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8, zero_padding=zero_padding)
    _sentinel_buffers(b, fp8)
    idx_d, x_d, w_d = dev(idx), dev_bf16(x), dev(w)
    if path == "fused":
        b.layout_dispatch(x_d, idx_d, w_d)
    elif path == "dispatch":
        b.layout(idx_d)
        b.dispatch(x_d, idx_d, w_d)
    elif path == "fp8_input":
        q = oracle.dispatch(x, np.zeros((T, 1), np.int32), None, 1, 1, fp8=True, capacity=T)
        b.layout(idx_d)
        b.dispatch_fp8_input(dev(q["recv_x"][:T]), dev(q["recv_scales"][:T]), idx_d, w_d)
    else:
        b.layout(idx_d)
        b.dispatch_ranked(x_d, idx_d, w_d)
        b.expand()
    b.check_status()
    lay = oracle.layout(idx, E, R, A)
    do = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=b.capacity)
    rows_used = int(lay["expert_offsets"][-1])
    if shape == "alignment_example":
        assert list(lay["expert_offsets"]) == [0, 4, 8]
    _check_padding(b, do, fp8, zero_padding, rows_used, lay["num_tokens_per_expert"],
                   lay["expert_offsets"])
    assert np.array_equal(b.tok_slot_row.cpu().numpy(), do["tok_slot_row"])


# --------------------------------------------------------------------------
# workspace that does not hold this configuration's layout
# --------------------------------------------------------------------------

def _guarded(b, fp8, H):
    """Replace the receive rows, scales and sources by views that start one
    row into larger tensors, with sentinel guard rows around them."""
    cap = b.capacity
    if fp8:
        big = torch.full((cap + 2, H), SENTINEL, dtype=torch.uint8, device="cuda")
        bigs = torch.full((cap + 2, H // 128), 3.0, dtype=torch.float32, device="cuda")
        b.recv_scales = bigs[1:cap + 1]
    else:
        big = torch.full((cap + 2, H), 3.0, dtype=torch.bfloat16, device="cuda")
        bigs = None
    b.recv_x = big[1:cap + 1]
    bsrc = torch.full((cap + 2,), -7, dtype=torch.int32, device="cuda")
    b.row_src = bsrc[1:cap + 1]
    return big, bigs, bsrc


def _guards_intact(big, bigs, bsrc, fp8):
    g = [big[0], big[-1]]
    want = SENTINEL if fp8 else 3.0
    assert all(torch.all(r == want).item() for r in g)
    if bigs is not None:
        assert torch.all(bigs[0] == 3.0).item() and torch.all(bigs[-1] == 3.0).item()
    assert bsrc[0].item() == -7 and bsrc[-1].item() == -7


@pytest.mark.parametrize("fp8", [False, True])
def test_padding_fill_with_a_workspace_of_no_layout(fp8):
    """A prepared workspace that no layout has written, its count section
    all ones (-1) and the segment starts garbage: nothing is written and the
    workspace bit is set."""
    T, H, k, E, R, A = 100, 256, 4, 16, 4, 4
    idx, x, w = _case(45, T, H, k, E, R)
    say(f"pad fill, no layout, fp8={fp8}")
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    big, bigs, bsrc = _guarded(b, fp8, H)
    b.workspace[256:].fill_(0xFF)
    b.expert_offsets.copy_(torch.arange(-3, E - 2, dtype=torch.int32, device="cuda") * 1000)
    before = big.clone()
    b.dispatch(dev_bf16(x), dev(idx), dev(w))
    assert _status_of(b) == ep.EP_ERR_WORKSPACE
    _guards_intact(big, bigs, bsrc, fp8)
    assert torch.equal(big, before)                   # nothing written at all
    assert torch.all(bsrc[1:-1] == -7).item()


@pytest.mark.parametrize("fp8", [False, True])
def test_padding_fill_with_garbage_counts_stays_in_bounds(fp8):
    """A layout of this configuration ran, then its workspace counts and
    ranks were overwritten with all ones (-1): the header still matches, and
    every write stays inside the receive rows."""
    T, H, k, E, R, A = 100, 256, 4, 16, 4, 4
    idx, x, w = _case(46, T, H, k, E, R)
    say(f"pad fill, garbage counts, fp8={fp8}")
    b = ep.EpBuffers(T, H, k, E, R, A, fp8=fp8)
    big, bigs, bsrc = _guarded(b, fp8, H)
    b.layout(dev(idx))
    torch.cuda.synchronize()
    b.workspace[256:].fill_(0xFF)
    b.dispatch(dev_bf16(x), dev(idx), dev(w))
    _status_of(b)  # any status: only the bounds are checked here
    _guards_intact(big, bigs, bsrc, fp8)
    # the same with segment starts pushed past the buffer's end
    b.expert_offsets.copy_(torch.full((E + 1,), b.capacity - 1, dtype=torch.int32,
                                      device="cuda"))
    b.dispatch(dev_bf16(x), dev(idx), dev(w))
    _status_of(b)
    _guards_intact(big, bigs, bsrc, fp8)


# --------------------------------------------------------------------------
# a dispatch given another route than its layout's
# --------------------------------------------------------------------------

def _other_route(idx, E):
    """idx with token 5's first slot moved to an expert it does not hold and
    token 9's second slot masked: the same configuration, another route."""
    other = idx.copy()
    held = set(int(e) for e in idx[5])
    other[5, 0] = next(e for e in range(E) if e not in held)
    other[9, 1] = -1
    return other


@pytest.mark.parametrize("path", ["dispatch_bf16", "dispatch_fp8", "fp8_input", "ranked"])
def test_dispatch_with_another_route_is_reported(path):
    """The layout records each selection's expert in the workspace; a
    dispatch given a different route with the same sizes sets the workspace
    status bit, gives the two changed selections no row, and places every
    other selection where the layout's route puts it."""
    T, H, k, E, R = 300, 256, 4, 16, 4
    rng = np.random.default_rng(55)
    idx = W.random_routes(rng, T, E, k)
    x = W.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    other = _other_route(idx, E)
    fp8 = path in ("dispatch_fp8", "fp8_input")
    b = ep.EpBuffers(T, H, k, E, R, 1, fp8=fp8)
    b.status.zero_()
    b.layout(dev(idx))
    say(f"another route through {path}")
    if path == "ranked":
        b.dispatch_ranked(dev_bf16(x), dev(other), dev(w))
    elif path == "fp8_input":
        codes = rng.integers(0, 256, (T, H), dtype=np.uint8)
        scales = rng.random((T, H // 128)).astype(np.float32)
        b.dispatch_fp8_input(dev(codes), dev(scales), dev(other), dev(w))
    else:
        b.dispatch(dev_bf16(x), dev(other), dev(w))
    assert _status_of(b) == ep.EP_ERR_WORKSPACE
    if path == "ranked":
        return
    do = oracle.dispatch(x, idx, w, E, R, capacity=T * k)
    tsr = b.tok_slot_row.cpu().numpy()
    changed = np.zeros((T, k), bool)
    changed[5, 0] = changed[9, 1] = True
    assert np.all(tsr[changed] == -1)
    assert np.array_equal(tsr[~changed], do["tok_slot_row"][~changed])
