"""Pins for the oracle's arithmetic readings: the exact form of the FP8
block quantiser, and the slot order and fused multiply-add form of every
fixed-order fp32 sum.

The pages fix the FP8 rule as one fp32 scale per 128 values with
scale = amax / 448 rounded to nearest even ("Deep Dive - DeepEP",
"Precision: FP8 on the wire, BF16 for the reduction"), and combine as an
fp32 accumulation rounded to bf16 once ("Deep Dive - DeepEP", "Combine:
reverse routing plus reduction").  Where they leave the form open, the
readings are: codes are E4M3(fp32(x / scale)), a correctly rounded
division; the terms of a token are summed in slot order j = 0..k-1 from +0;
a gated term is one fused multiply-add.

The expected values below come from outside the oracle: numpy's IEEE fp32
division, torch's float8_e4m3fn conversion, and sums worked out by hand
(closed forms), each chosen so that another reading gives another result.
"""
import numpy as np

import oracle
from tests.ep_cases import bf16_bits_exact, bits_to_f32


def _fp8_one_block_per_token(x_bits):
    T, H = x_bits.shape
    idx = np.zeros((T, 1), np.int32)
    d = oracle.dispatch(x_bits, idx, None, 1, 1, fp8=True)
    # with one expert and one slot, token t lands on row t
    assert np.array_equal(d["tok_slot_row"][:, 0], np.arange(T))
    return d["recv_x"][:T], d["recv_scales"][:T]


def _expected_codes(x_bits, scale):
    """torch's E4M3 rounding of numpy's fp32 x / scale per block (scale
    broadcast over the block's 128 values).  A scale that underflows to 0
    (amax below 448 * 2^-150) gives zero codes, and a quotient above 448,
    which only a subnormal scale allows, saturates to 448 (the saturation
    rule is pinned on its own in test_oracle_pins)."""
    import torch

    xv = bits_to_f32(x_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = xv / scale
    q = np.where(scale > 0, np.clip(q, np.float32(-448.0), np.float32(448.0)), np.float32(0.0))
    codes = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.where(scale > 0, codes, np.uint8(0)).astype(np.uint8)


def test_fp8_scale_is_the_rounded_quotient_for_every_bf16_amax():
    """Every positive finite bf16 value as a block's amax: the scale's bits
    equal numpy's correctly rounded fp32 amax / 448.  Multiplying by a
    rounded 1/448 instead differs for about half of these amaxes."""
    amax_bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    n = amax_bits.size
    rng = np.random.default_rng(11)
    amax = bits_to_f32(amax_bits)
    # the rest of the block: random magnitudes below amax, random signs,
    # rounded down to bf16 so that none exceeds it
    frac = rng.random((n, 127)).astype(np.float32)
    rest = (amax[:, None] * frac).astype(np.float32)
    rest_bits = (rest.view(np.uint32) >> 16).astype(np.uint16)
    rest_bits |= (rng.random((n, 127)) < 0.5).astype(np.uint16) << 15
    pos = rng.integers(0, 128, n)
    x = np.empty((n, 128), np.uint16)
    for i in range(n):
        x[i] = np.insert(rest_bits[i], pos[i], amax_bits[i] | (0x8000 if i % 3 == 0 else 0))
    codes, scales = _fp8_one_block_per_token(x)
    want = np.float32(amax) / np.float32(448.0)
    assert scales.dtype == np.float32
    assert np.array_equal(scales[:, 0].view(np.uint32), want.view(np.uint32))
    # and the codes of every block: torch's E4M3 of numpy's fp32 x / scale
    assert np.array_equal(codes, _expected_codes(x, want[:, None]))


def test_fp8_codes_are_e4m3_of_the_rounded_quotient():
    """Codes of normal data (the workloads' N(0, sigma^2) rows, several
    blocks per token): torch's E4M3 rounding of numpy's correctly rounded
    fp32 x / scale.  Multiplying x by 448 / amax instead of dividing by the
    scale changes a few codes per ten thousand here."""
    rng = np.random.default_rng(12)
    T, H = 512, 4096
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf *= np.float32(2.0) ** rng.integers(-20, 20, (T, 1)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)  # truncation keeps finite bf16
    codes, scales = _fp8_one_block_per_token(x)
    xb = x.reshape(T, H // 128, 128)
    amax = np.abs(bits_to_f32(xb)).max(axis=2)
    want_scale = amax / np.float32(448.0)
    assert np.array_equal(scales.view(np.uint32), want_scale.view(np.uint32))
    assert np.array_equal(codes.reshape(T, H // 128, 128),
                          _expected_codes(xb, want_scale[:, :, None]))


# --------------------------------------------------------------------------
# slot order: terms 1, 2^24, -2^24 (exact in bf16).  From +0 in this order
# the sum is 0: 1 + 2^24 is a tie between 2^24 and 2^24 + 2 and rounds to
# the even 2^24, and 2^24 - 2^24 = 0.  In the reverse order it is 1.
# --------------------------------------------------------------------------

def _order_rows():
    return bf16_bits_exact(np.array([[1.0], [2.0 ** 24], [-(2.0 ** 24)]], np.float32))


def test_combine_sums_in_slot_order():
    y = _order_rows()
    fwd = np.array([[0, 1, 2]], np.int32)
    rev = np.array([[2, 1, 0]], np.int32)
    for w in (None, np.ones((1, 3), np.float32)):
        out, acc = oracle.combine(y, fwd, w)
        assert acc[0, 0] == 0.0 and out[0, 0] == 0
        out, acc = oracle.combine(y, rev, w)
        assert acc[0, 0] == 1.0 and bits_to_f32(out)[0, 0] == 1.0
    # a masked slot in between changes nothing
    out, acc = oracle.combine(y, np.array([[0, -1, 1, 2]], np.int32), None)
    assert acc[0, 0] == 0.0


def test_dispatch_backward_sums_in_slot_order():
    g = _order_rows()
    out, acc = oracle.dispatch_backward(g, np.array([[0, 1, 2]], np.int32))
    assert acc[0, 0] == 0.0 and out[0, 0] == 0
    out, acc = oracle.dispatch_backward(g, np.array([[2, 1, 0]], np.int32))
    assert acc[0, 0] == 1.0 and bits_to_f32(out)[0, 0] == 1.0


def _one_rank_slice(tsr):
    """A non-expanded handle for one token whose slots all live on the one
    rank (local expert = slot, all three valid)."""
    k = tsr.shape[1]
    return dict(rank_token_offsets=np.array([0, 1], np.int32),
                recv_topk_idx=np.arange(k, dtype=np.int32).reshape(1, k),
                recv_topk_weights=np.ones((1, k), np.float32),
                recv_src=np.zeros(1, np.int32), tok_rank_row=np.zeros((1, 1), np.int32))


def test_ranked_stage_one_sums_in_slot_order():
    y = _order_rows()
    for weighted in (False, True):
        tsr = np.array([[0, 1, 2]], np.int32)
        out, acc, part = oracle.combine_ranked(y, tsr, _one_rank_slice(tsr), weighted)
        assert part[0, 0] == 0.0 and acc[0, 0] == 0.0 and out[0, 0] == 0
        tsr = np.array([[2, 1, 0]], np.int32)
        out, acc, part = oracle.combine_ranked(y, tsr, _one_rank_slice(tsr), weighted)
        assert part[0, 0] == 1.0 and acc[0, 0] == 1.0


# --------------------------------------------------------------------------
# fused multiply-add: slot 0 holds y = 1 with gate g0 = -(1 + 2^-7 + 2^-23);
# slot 1 holds y = 1 + 2^-7 (exact in bf16) with gate 1 + 2^-23.  The exact
# product of slot 1 is 1 + 2^-7 + 2^-23 + 2^-30, so one fused multiply-add
# onto g0 leaves exactly 2^-30; rounding the product to fp32 first (it drops
# the 2^-30) and then adding leaves 0.
# --------------------------------------------------------------------------

def _fma_case():
    y = bf16_bits_exact(np.array([[1.0], [1.0 + 2.0 ** -7]], np.float32))
    g0 = np.float32(-(1.0 + 2.0 ** -7 + 2.0 ** -23))
    g1 = np.float32(1.0 + 2.0 ** -23)
    assert float(g0) == -(1.0 + 2.0 ** -7 + 2.0 ** -23) and float(g1) == 1.0 + 2.0 ** -23
    return y, np.array([[g0, g1]], np.float32)


def test_combine_term_is_one_fused_multiply_add():
    y, w = _fma_case()
    out, acc = oracle.combine(y, np.array([[0, 1]], np.int32), w)
    assert float(acc[0, 0]) == 2.0 ** -30
    assert float(bits_to_f32(out)[0, 0]) == 2.0 ** -30  # a power of two: exact in bf16


def test_ranked_stage_one_term_is_one_fused_multiply_add():
    y, w = _fma_case()
    tsr = np.array([[0, 1]], np.int32)
    ne = _one_rank_slice(tsr)
    ne["recv_topk_weights"] = w.copy()
    out, acc, part = oracle.combine_ranked(y, tsr, ne, True)
    assert float(part[0, 0]) == 2.0 ** -30 and float(acc[0, 0]) == 2.0 ** -30


def test_combine_starts_from_positive_zero():
    """A single term of -0 gives +0 (the sum starts at +0, and +0 + -0 is
    +0); starting from the first term would give -0."""
    y = bf16_bits_exact(np.array([[-0.0]], np.float32))
    out, acc = oracle.combine(y, np.array([[0]], np.int32), None)
    assert out[0, 0] == 0x0000 and not np.signbit(acc[0, 0])
    out, acc = oracle.combine(y, np.array([[0]], np.int32), np.ones((1, 1), np.float32))
    assert out[0, 0] == 0x0000
    out, acc = oracle.dispatch_backward(y, np.array([[0]], np.int32))
    assert out[0, 0] == 0x0000


def test_dispatch_rejects_non_finite_gates_of_used_selections():
    """A used selection's gate must be finite ("Deep Dive - DeepEP", "A
    runnable routing ledger" rejects an invalid gate weight); an unused
    selection's gate is never read, so NaN there is accepted.  Negative
    gates are accepted (the reading: combine is linear in the gate)."""
    import pytest

    x = np.zeros((2, 128), np.uint16)
    idx = np.array([[0, -1], [2, 3]], np.int32)
    for bad in (np.inf, -np.inf, np.nan):
        w = np.full((2, 2), 0.5, np.float32)
        w[1, 1] = bad
        for call in (lambda: oracle.dispatch(x, idx, w, 4, 2),
                     lambda: oracle.dispatch(x, idx, w, 4, 2, fp8=True),
                     lambda: oracle.dispatch_fp8_input(np.zeros((2, 128), np.uint8),
                                                       np.ones((2, 1), np.float32), idx, w, 4, 2),
                     lambda: oracle.dispatch_ranked(x, idx, w, 4, 2)):
            with pytest.raises(oracle.OracleError) as e:
                call()
            assert e.value.code == oracle.BAD_ARG
    w = np.array([[-0.5, np.nan], [0.25, 0.75]], np.float32)  # NaN only in the unused slot
    d = oracle.dispatch(x, idx, w, 4, 2)
    assert d["recv_weights"][d["tok_slot_row"][0, 0]] == np.float32(-0.5)
    oracle.dispatch_ranked(x, idx, w, 4, 2)
