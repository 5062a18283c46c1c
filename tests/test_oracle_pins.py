"""Pins for the CPU oracle: values the pages print, closed forms, special
cases that reduce to a library routine, and brute force on tiny inputs.

Every check here is independent of the oracle's own code path: printed
numbers from the pages (tests/golden/), exhaustive enumeration, numpy's
lexsort, torch's float8 / bfloat16 conversions, or exact fp64 sums.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from ep_workloads import random_routes
from tests.ep_cases import Ledger, bf16_bits_exact, bits_to_f32, row_experts
from tests.golden_fixtures import load


class OracleBackend:
    hidden_multiple = 1

    def layout(self, idx, E, R, A):
        return oracle.layout(idx, E, R, A)

    def dispatch(self, x, idx, w, E, R, A, fp8, cap):
        return oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=cap)

    def combine(self, y, tsr, w):
        return oracle.combine(y, tsr, w)[0]


BE = OracleBackend()


# --------------------------------------------------------------------------
# bf16 rounding ("Deep Dive - DeepEP", "Combine: reverse routing plus reduction")
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_random_and_ties():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(100),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-30),
        # exact ties: low 16 bits == 0x8000, both parities of the kept lsb
        (rng.integers(0x3F000000, 0x47000000, 4000, dtype=np.uint32) & 0xFFFF0000 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 257.0, 3.0e38, -3.0e38], np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(v), ref)


def test_bf16_cancellation_example(golden):
    fx = golden("cancellation.txt")
    c = fx.nums("contributions")
    # Two-stage: bf16 subtotal of the first two, then the rest.
    sub = bits_to_f32(oracle.bf16_round(np.float32(c[0]) + np.float32(c[1])))
    assert sub == fx.num("bf16_subtotal_of_first_two")
    two = bits_to_f32(oracle.bf16_round(np.float32(sub) + np.float32(c[2])))
    assert two == fx.num("bf16_subtotal_then_rest")
    # Through oracle combine: one token, three pre-weighted rows, one bf16 cast.
    y = bf16_bits_exact(np.array(c, np.float32).reshape(3, 1))
    tsr = np.array([[0, 1, 2]], np.int32)
    out, acc = oracle.combine(y, tsr, None)
    assert bits_to_f32(out)[0, 0] == fx.num("fp32_sum_then_bf16")
    # Same with explicit unit gates (three fused multiply-adds).
    out1, _ = oracle.combine(y, tsr, np.ones((1, 3), np.float32))
    assert bits_to_f32(out1)[0, 0] == fx.num("fp32_sum_then_bf16")


# --------------------------------------------------------------------------
# FP8 E4M3FN ("Deep Dive - DeepEP", "Precision: FP8 on the wire, ...")
# --------------------------------------------------------------------------

def test_e4m3_code_table_closed_forms():
    vals = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    assert vals[0x01] == 2.0 ** -9 and vals[0x07] == 7 * 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6 and vals[0x38] == 1.0
    assert math.isnan(vals[0x7F]) and math.isnan(vals[0xFF])
    assert vals[0x80] == 0.0 and math.copysign(1, vals[0x80]) < 0
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be increasing"
    # library routine: torch's float8_e4m3fn decoding of every non-NaN code
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(lib, vals[codes])


def test_e4m3_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_value(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_midpoints_round_to_even_code():
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        assert float(mid) == (vals[c] + vals[c + 1]) / 2  # exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == even, c
        assert oracle.e4m3_encode(np.array([-mid]))[0] == 0x80 | even, c
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1000))
        assert oracle.e4m3_encode(np.array([below]))[0] == c
        assert oracle.e4m3_encode(np.array([above]))[0] == c + 1


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(50000).astype(np.float32) * np.float32(50),
        rng.uniform(-448, 448, 20000).astype(np.float32),
        rng.standard_normal(20000).astype(np.float32) * np.float32(0.01),  # subnormal codes
        np.array([0.0, -0.0, -1e-7, 1e-7, 448.0, -448.0, 447.9, 2.0 ** -10], np.float32),
    ])
    v = v[np.abs(v) <= 448]
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), lib)


def test_e4m3_saturates():
    v = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, -1e30], np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E] * 5 + [0x7E, 0xFE]


def test_fp8_row_bytes(golden):
    fx = golden("fp8_row_bytes.txt")
    H = fx.num("hidden", int)
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((1, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    idx = np.array([[0]], np.int32)
    d = oracle.dispatch(x, idx, np.ones((1, 1), np.float32), 1, 1, fp8=True)
    assert d["recv_x"].dtype == np.uint8 and d["recv_x"].shape[1] == fx.num("fp8_payload_bytes", int)
    assert d["recv_scales"].shape[1] * 4 == fx.num("fp8_scale_bytes", int)
    assert H // fx.num("values_per_scale", int) == d["recv_scales"].shape[1]
    assert x.shape[1] * 2 == fx.num("bf16_row_bytes", int)


def test_fp8_quantisation_properties():
    """Per 128-value block: the largest magnitude maps to code 448 (0x7E);
    dequantised values lie within half an e4m3 step of x; a block of zeros
    gets scale 0 and zero codes; a wrong block size or divisor fails these."""
    rng = np.random.default_rng(3)
    H = 512
    xf = rng.standard_normal((3, H)).astype(np.float32)
    xf[1, 128:256] *= 1e-3           # a quiet block (many subnormal codes)
    xf[2, 256:384] = 0.0             # an all-zero block
    xf[2, 300] = -0.0
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)
    xv = bits_to_f32(xb).reshape(3, H // 128, 128).astype(np.float64)
    idx = np.array([[0], [0], [0]], np.int32)
    d = oracle.dispatch(xb, idx, None, 1, 1, fp8=True)
    q = d["recv_x"][:3].reshape(3, H // 128, 128)
    s = d["recv_scales"][:3].astype(np.float64)
    for t in range(3):
        for b in range(H // 128):
            blk = xv[t, b]
            amax = np.abs(blk).max()
            if amax == 0:
                assert s[t, b] == 0 and np.all(q[t, b] == 0)
                continue
            # the rounded fp32 quotient, bit for bit (numpy's IEEE division)
            assert np.float32(s[t, b]) == np.float32(amax) / np.float32(448.0)
            assert (q[t, b] & 0x7F).max() == 0x7E
            deq = oracle.e4m3_value(q[t, b]) * s[t, b]
            mag = np.abs(blk) / s[t, b]
            step = np.where(mag < 2.0 ** -6, 2.0 ** -9,
                            2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))
            assert np.all(np.abs(deq - blk) <= (step / 2) * s[t, b] * (1 + 1e-6))
            assert np.all(np.sign(deq[blk != 0]) == np.sign(blk[blk != 0]))


# --------------------------------------------------------------------------
# layout / placement
# --------------------------------------------------------------------------

def test_t0_example_layout_and_combine(golden):
    fx = golden("t0_example.txt")
    idx = np.array([fx.nums(f"route.{t}", int) for t in ("T0", "T1", "T2")], np.int32)
    E, R = fx.num("num_experts", int), fx.num("num_ranks", int)
    lay = oracle.layout(idx, E, R)
    assert list(lay["num_tokens_per_expert"]) == fx.nums("counts", int)
    assert list(lay["expert_offsets"]) == fx.nums("offsets", int)
    assert list(lay["num_tokens_per_rank"]) == fx.nums("distinct_tokens_per_rank", int)
    # Combine recovers 0.73 x Expert2(T0) + 0.27 x Expert7(T0): with expert e
    # scaling its row by (e + 1) and x[T0] = 1, that is 0.73*3 + 0.27*8.
    g = fx.nums("gates.T0")
    w = np.array([g, [0.5, 0.5], [0.5, 0.5]], np.float32)
    x = bf16_bits_exact(np.ones((3, 4), np.float32))
    d = oracle.dispatch(x, idx, w, E, R)
    off = lay["expert_offsets"]
    seg7 = d["row_src"][off[7]:off[8]] // 2
    assert list(seg7) == fx.nums("expert7_tokens", int)
    rexp = row_experts(off, int(off[-1]))
    y = np.zeros((6, 4), np.float32)
    y[: off[-1]] = (rexp[:, None] + 1) * bits_to_f32(d["recv_x"][: off[-1]])
    out, acc = oracle.combine(bf16_bits_exact(y), d["tok_slot_row"], w)
    want = g[0] * 3 + g[1] * 8
    assert abs(acc[0, 0] - want) <= 4 * 2.0 ** -24 * want
    swapped = g[1] * 3 + g[0] * 8
    assert abs(acc[0, 0] - swapped) > 1.0


def test_layout_fragment(golden):
    fx = golden("layout_fragment.txt")
    n2, n3 = fx.num("expert2_count", int), fx.num("expert3_count", int)
    idx = np.array([[2]] * n2 + [[3]] * n3, np.int32)
    lay = oracle.layout(idx, 4, 1)
    assert lay["expert_offsets"][2] == fx.num("expert2_offset", int)
    assert lay["expert_offsets"][3] == fx.num("expert3_offset", int)
    x = bf16_bits_exact(np.arange(n2 + n3, dtype=np.float32)[:, None] * np.ones((1, 2), np.float32))
    d = oracle.dispatch(x, idx, None, 4, 1)
    # dst = prefix[expert]++: rows handed out in token order from the offset
    assert list(d["tok_slot_row"][:, 0]) == list(range(n2 + n3))


def test_alignment_example(golden):
    fx = golden("alignment.txt")
    c = fx.nums("counts", int)
    A = fx.num("alignment", int)
    idx = np.array([[0]] * c[0] + [[1]] * c[1], np.int32)
    lay = oracle.layout(idx, 2, 1, A)
    off = lay["expert_offsets"]
    assert list(off[:2]) == fx.nums("starts", int)
    assert list(off[:2] + lay["num_tokens_per_expert"]) == fx.nums("ends", int)
    assert off[2] == fx.num("total_slots", int)
    assert list(lay["num_tokens_per_expert"]) == fx.nums("unaligned_counts", int)
    x = bf16_bits_exact(np.full((sum(c), 8), 3.0, np.float32))
    d = oracle.dispatch(x, idx, np.ones((sum(c), 1), np.float32), 2, 1, A, capacity=8)
    pad = [p for p in range(8) if not (0 <= p < 3 or 4 <= p < 5)]
    assert all(d["row_src"][p] == -1 for p in pad)
    assert all(d["recv_weights"][p] == 0 for p in pad)
    assert np.all(d["recv_x"][pad] == 0)


def test_expected_destinations_by_enumeration(golden):
    """Feed every k-subset of experts as one token: the mean number of distinct
    destination ranks per token is the page's 1.666667 (and the closed form)."""
    fx = golden("expected_destinations.txt")
    E, R, k = (fx.num(n, int) for n in ("num_experts", "num_ranks", "num_topk"))
    idx = np.array(list(itertools.combinations(range(E), k)), np.int32)
    lay = oracle.layout(idx, E, R)
    per_token = lay["is_token_in_rank"].sum(axis=1)
    assert (per_token == 1).sum() == fx.num("pairs_single_rank", int)
    assert (per_token == R).sum() == fx.num("pairs_both_ranks", int)
    mean = lay["num_tokens_per_rank"].sum() / len(idx)
    assert round(mean, 6) == fx.num("expected_destinations")
    closed = R * (1 - math.comb(E - E // R, k) / math.comb(E, k))
    assert abs(mean - closed) < 1e-12
    # a larger case by enumeration against the same closed form
    E, R, k = 8, 4, 3
    idx = np.array(list(itertools.combinations(range(E), k)), np.int32)
    lay = oracle.layout(idx, E, R)
    closed = R * (1 - math.comb(E - E // R, k) / math.comb(E, k))
    assert abs(lay["num_tokens_per_rank"].sum() / len(idx) - closed) < 1e-12


@pytest.mark.parametrize("seed", range(40))
def test_placement_brute_force(seed):
    """Positions against an independent ranking: sort valid (expert, token)
    pairs with numpy's lexsort and lay the segments out at aligned starts."""
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(0, 17))
    R = int(rng.choice([1, 2, 4]))
    E = R * int(rng.integers(1, 5))
    k = int(rng.integers(1, min(E, 3) + 1))
    A = int(rng.choice([1, 2, 4]))
    idx = random_routes(rng, T, E, k, mask_prob=0.2)
    lay = oracle.layout(idx, E, R, A)
    x = (rng.integers(0, 0x7F00, (T, 3), dtype=np.uint16))
    w = rng.random((T, k)).astype(np.float32)
    d = oracle.dispatch(x, idx, w, E, R, A)

    t_of, j_of = np.nonzero(idx >= 0)
    e_of = idx[t_of, j_of]
    order = np.lexsort((t_of, e_of))  # by expert, then token
    counts = np.bincount(e_of, minlength=E)
    padded = -(-counts // A) * A
    starts = np.concatenate([[0], np.cumsum(padded)])
    assert np.array_equal(lay["expert_offsets"], starts)
    assert np.array_equal(lay["num_tokens_per_expert"], counts)
    expect = np.full((T, k), -1, np.int64)
    for rank_in_e, n in enumerate(order):
        e = e_of[n]
        first = np.searchsorted(e_of[order], e)
        expect[t_of[n], j_of[n]] = starts[e] + (rank_in_e - first)
    assert np.array_equal(d["tok_slot_row"], expect)
    # distinct tokens per rank, by sets
    ranks = [set() for _ in range(R)]
    for t, j in zip(t_of, j_of):
        ranks[idx[t, j] // (E // R)].add(t)
    assert list(lay["num_tokens_per_rank"]) == [len(s) for s in ranks]
    assert np.array_equal(lay["rank_offsets"], starts[np.arange(R + 1) * (E // R)])
    # rows are bit copies of their source token, weights follow the row
    for t, j in zip(t_of, j_of):
        p = expect[t, j]
        assert np.array_equal(d["recv_x"][p], x[t])
        assert d["row_src"][p] == t * k + j
        assert d["recv_weights"][p] == w[t, j]


def test_route_validation():
    x = np.zeros((2, 8), np.uint16)
    for bad in ([[0, 0], [1, 2]], [[0, 4], [1, 2]], [[-2, 1], [1, 2]]):
        with pytest.raises(oracle.OracleError) as e:
            oracle.layout(np.array(bad, np.int32), 4, 2)
        assert e.value.code == oracle.BAD_ROUTE
        with pytest.raises(oracle.OracleError):
            oracle.dispatch(x, np.array(bad, np.int32), None, 4, 2)
    with pytest.raises(oracle.OracleError) as e:
        oracle.layout(np.zeros((2, 2), np.int32), 6, 4)  # E % R != 0
    assert e.value.code == oracle.BAD_ARG
    with pytest.raises(oracle.OracleError) as e:  # capacity too small
        oracle.dispatch(x, np.array([[0, 1], [2, 3]], np.int32), None, 4, 2, capacity=3)
    assert e.value.code == oracle.NO_CAPACITY
    with pytest.raises(oracle.OracleError) as e:  # FP8 needs H % 128 == 0
        oracle.dispatch(x, np.array([[0, 1], [2, 3]], np.int32), None, 4, 2, fp8=True)
    assert e.value.code == oracle.BAD_ARG
    xi = x.copy()
    xi[0, 0] = 0x7F80  # +inf
    with pytest.raises(oracle.OracleError) as e:
        oracle.dispatch(xi, np.array([[0, 1], [2, 3]], np.int32), None, 4, 2)
    assert e.value.code == oracle.BAD_ARG


def test_empty_batch():
    lay = oracle.layout(np.zeros((0, 2), np.int32), 4, 2)
    assert list(lay["expert_offsets"]) == [0] * 5
    d = oracle.dispatch(np.zeros((0, 8), np.uint16), np.zeros((0, 2), np.int32), None, 4, 2)
    assert d["tok_slot_row"].shape == (0, 2)
    out, _ = oracle.combine(np.zeros((1, 8), np.uint16), np.zeros((0, 2), np.int32), None)
    assert out.shape == (0, 8)


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

def test_four_token_ledger(golden):
    L = Ledger()
    idx, w = L.routes()
    r = L.run(BE, idx, w)
    for i, t in enumerate(L.tokens):
        want = np.array(L.fx.nums(f"expect.{t}"))
        assert np.all(np.abs(r["out"][i] - want) <= 0.005 + 2.0 ** -7 * np.abs(want)), t
    # receive order and local / remote of each expert's copies
    d, off = r["dispatch"], r["layout"]["expert_offsets"]
    src_rank = L.fx.nums("source_rank", int)
    for e in range(L.E):
        got = []
        for p in range(off[e], off[e + 1]):
            t = d["row_src"][p] // 2
            where = "local" if src_rank[t] == e // (L.E // L.R) else "remote"
            got.append(f"{L.tokens[t]}:{where}")
        assert got == L.fx[f"expert.{e}"]
    assert (d["row_src"][: r["rows_used"]] >= 0).sum() == L.fx.num("inverse_entries", int)
    r4 = L.run(BE, idx, w, alignment=4)
    assert r4["rows_used"] == L.fx.num("slots_at_alignment_4", int)
    assert np.array_equal(r4["out"], r["out"])


def test_ledger_variants(golden):
    L = Ledger()
    v = L.var
    idx, w = L.routes({"a": v["same_rank.route.a"]})
    r = L.run(BE, idx, w)
    assert r["layout"]["num_tokens_per_expert"].sum() == v.num("same_rank.assignments", int)
    assert r["layout"]["num_tokens_per_rank"].sum() == v.num("same_rank.destination_rows", int)
    assert abs(r["out"][0, 0] - v.num("same_rank.expect.a0")) <= 0.005 + 2.0 ** -7 * 3.3
    idx, w = L.routes({"a": v["masked.route.a"]})
    w[0, 1] = np.nan  # an unused slot's gate must never be read
    r = L.run(BE, idx, w)
    assert r["layout"]["num_tokens_per_expert"].sum() == v.num("masked.assignments", int)
    assert r["layout"]["num_tokens_per_rank"].sum() == v.num("masked.destination_rows", int)
    want = np.array(v.nums("masked.expect.a"))
    assert np.all(np.abs(r["out"][0] - want) <= 0.005 + 2.0 ** -7 * np.abs(want))


def test_weight_applied_exactly_once(golden):
    fx = golden("weight_applied_once.txt")
    g = np.array([fx.nums("gates")], np.float32)
    raw = np.array([fx.nums("raw.0"), fx.nums("raw.1")], np.float32)
    tsr = np.array([[0, 1]], np.int32)
    y_raw = bf16_bits_exact(raw)
    y_w = torch.from_numpy(g.T * raw).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def close(out, key):
        want = np.array(fx.nums(key))
        return np.all(np.abs(bits_to_f32(out)[0] - want) <= 0.005 + 2.0 ** -7 * np.abs(want))

    assert close(oracle.combine(y_raw, tsr, g)[0], "weighted_once")       # gate in combine
    assert close(oracle.combine(y_w, tsr, None)[0], "weighted_once")      # caller weighted
    assert close(oracle.combine(y_raw, tsr, None)[0], "raw_sum")          # never weighted
    assert close(oracle.combine(y_w, tsr, g)[0], "weighted_twice")        # weighted twice


def test_combine_against_exact_fp64_sum():
    """The fp32 fixed-order accumulator is within k rounding errors of the
    exact (fp64) weighted sum, and the output is its bf16 rounding (torch)."""
    rng = np.random.default_rng(5)
    T, H, k, cap = 50, 64, 6, 400
    y = (rng.standard_normal((cap, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    tsr = rng.integers(-1, cap, (T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out, acc = oracle.combine(y, tsr, w)
    yf = bits_to_f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    mag = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if tsr[t, j] >= 0:
                exact[t] += np.float64(w[t, j]) * yf[tsr[t, j]]
                mag[t] += abs(np.float64(w[t, j])) * np.abs(yf[tsr[t, j]])
    assert np.all(np.abs(acc - exact) <= k * 2.0 ** -24 * mag + 1e-45)
    lib = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, lib)


def test_combine_all_masked_token_is_positive_zero():
    y = bf16_bits_exact(np.ones((2, 8), np.float32))
    out, acc = oracle.combine(y, np.array([[-1, -1], [0, 1]], np.int32),
                              np.array([[np.nan, np.nan], [0.5, 0.5]], np.float32))
    assert np.all(out[0] == 0) and np.all(bits_to_f32(out[1]) == 1.0)


def test_adjoint_identity_fp64():
    """Combine (unrounded) is the adjoint of the weighted dispatch map:
    sum_t <combine(y)_t, u_t> == sum_p <y_p, w_src(p) u_src(p)>."""
    rng = np.random.default_rng(6)
    T, H, k, E, R = 40, 16, 3, 8, 2
    idx = random_routes(rng, T, E, k, mask_prob=0.1)
    w = rng.random((T, k)).astype(np.float32)
    x = np.zeros((T, H), np.uint16)
    d = oracle.dispatch(x, idx, w, E, R)
    cap = T * k
    y = (rng.standard_normal((cap, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    u = rng.standard_normal((T, H))
    _, acc = oracle.combine(y, d["tok_slot_row"], w)
    lhs = float((acc.astype(np.float64) * u).sum())
    yf = bits_to_f32(y).astype(np.float64)
    rhs = 0.0
    for p in range(int(oracle.layout(idx, E, R)["expert_offsets"][-1])):
        s = d["row_src"][p]
        t, j = divmod(int(s), k)
        rhs += float(np.dot(yf[p], np.float64(d["recv_weights"][p]) * u[t]))
    assert abs(lhs - rhs) <= 1e-5 * (np.abs(acc).sum() + 1)


@pytest.mark.parametrize("seed", range(8))
def test_fp8_input_dispatch_consistent_with_quantising_dispatch(seed):
    """Pre-quantised input: rows are the token's codes and scales, at the
    placement the brute-force test pins; quantising first and dispatching
    the codes gives the quantising dispatch's result bit for bit."""
    rng = np.random.default_rng(700 + seed)
    T, H, k, E, R = int(rng.integers(0, 40)), 256, 3, 8, 2
    A = int(rng.choice([1, 4]))
    idx = random_routes(rng, T, E, k, mask_prob=0.2)
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = rng.random((T, k)).astype(np.float32)
    q = oracle.dispatch(x, idx, w, E, R, A, fp8=True)
    # the token's own codes/scales: quantise it alone (one row, one expert)
    codes = np.zeros((T, H), np.uint8)
    scales = np.zeros((T, H // 128), np.float32)
    for t in range(T):
        one = oracle.dispatch(x[t:t + 1], np.array([[0]], np.int32), None, 1, 1, fp8=True)
        codes[t], scales[t] = one["recv_x"][0], one["recv_scales"][0]
    f = oracle.dispatch_fp8_input(codes, scales, idx, w, E, R, A)
    for key in ("recv_x", "recv_scales", "recv_weights", "tok_slot_row", "row_src"):
        assert np.array_equal(f[key], q[key]), key
    # random bytes (any code, any scale) travel unchanged
    rc = rng.integers(0, 256, (T, H), dtype=np.uint8)
    rs = rng.random((T, H // 128)).astype(np.float32)
    f = oracle.dispatch_fp8_input(rc, rs, idx, w, E, R, A)
    for t in range(T):
        for j in range(k):
            p = f["tok_slot_row"][t, j]
            if p >= 0:
                assert np.array_equal(f["recv_x"][p], rc[t]) and np.array_equal(f["recv_scales"][p], rs[t])
