"""Pins for the oracle's non-expanded (rank-deduplicated) path: the ledger's
printed row counts and outputs, the cancellation example staged per rank,
brute-force rank placement, agreement of expand(dispatch_ranked) with the
expanded dispatch, and the fp64 error bound of the two-stage sum."""
import numpy as np
import pytest

import oracle
from ep_workloads import random_routes
from tests.ep_cases import Ledger, bf16_bits_exact, bits_to_f32, row_experts


def _ledger_ne(routes_override=None):
    L = Ledger()
    idx, w = L.routes(routes_override)
    x = bf16_bits_exact(L.hidden)
    ne = oracle.dispatch_ranked(x, idx, w, L.E, L.R)
    return L, idx, w, x, ne


def test_ledger_rows_and_outputs(golden):
    L, idx, w, x, ne = _ledger_ne()
    # two selected experts always on different ranks: 8 rows for 8 slots
    assert ne["rank_token_offsets"][-1] == L.fx.num("inverse_entries", int)
    v = L.var
    L2, idx2, w2, x2, ne2 = _ledger_ne({"a": v["same_rank.route.a"]})
    assert ne2["rank_token_offsets"][-1] == v.num("same_rank.destination_rows", int)
    # token a travels once to rank 1 and carries both local experts there
    qa = ne2["tok_rank_row"][0, 1]
    assert ne2["tok_rank_row"][0, 0] == -1 and qa >= 0
    assert sorted(ne2["recv_topk_idx"][qa]) == [0, 1]
    ex = oracle.expand(ne2, 4, 2, L.E, L.R)
    assert (ex["row_src"][: 8] >= 0).sum() == v.num("same_rank.assignments", int)
    # the receiver's experts run on the expanded rows; combine via rank partials
    d = oracle.dispatch(x2, idx2, w2, L.E, L.R)
    used = 8
    rexp = row_experts(oracle.layout(idx2, L.E, L.R)["expert_offsets"], used)
    y = np.zeros((used, 2), np.float32)
    for p in range(used):
        y[p] = (rexp[p] + 1) * bits_to_f32(ex["recv_x"][p])
    out, acc, part = oracle.combine_ranked(bf16_bits_exact(y), ex["tok_slot_row"], ne2)
    assert abs(bits_to_f32(out)[0, 0] - v.num("same_rank.expect.a0")) <= 0.005 + 2.0 ** -7 * 3.3
    out_b, _, _ = oracle.combine_ranked(bf16_bits_exact(y), d["tok_slot_row"], ne2)
    assert np.array_equal(out, out_b)


def test_cancellation_staged_per_rank(golden):
    """256 and 1 on rank 0, -256 on rank 1: fp32 partials give 1 (a bf16
    subtotal of rank 0 would give 256 and the sum 0)."""
    fx = golden("cancellation.txt")
    c = fx.nums("contributions")
    idx = np.array([[0, 1, 2]], np.int32)   # experts 0, 1 on rank 0; 2 on rank 1 (E=4, R=2)
    x = bf16_bits_exact(np.ones((1, 8), np.float32))
    ne = oracle.dispatch_ranked(x, idx, None, 4, 2)
    ex = oracle.expand(ne, 1, 3, 4, 2)
    y = bf16_bits_exact(np.array(c, np.float32)[:, None] * np.ones((1, 8), np.float32))
    out, acc, part = oracle.combine_ranked(y, ex["tok_slot_row"], ne, weighted=False)
    assert np.all(bits_to_f32(out) == fx.num("fp32_sum_then_bf16"))
    assert np.all(part[ne["tok_rank_row"][0, 0]] == 257.0)
    sub = bits_to_f32(oracle.bf16_round(np.array([257.0], np.float32)))[0]
    assert fx.num("bf16_subtotal_of_first_two") == float(sub)


@pytest.mark.parametrize("seed", range(30))
def test_ranked_placement_brute_force_and_expand(seed):
    rng = np.random.default_rng(4000 + seed)
    T = int(rng.integers(0, 30))
    R = int(rng.choice([1, 2, 4]))
    E = R * int(rng.integers(1, 5))
    k = int(rng.integers(1, min(E, 4) + 1))
    A = int(rng.choice([1, 2, 4]))
    fp8 = bool(seed % 3 == 0)
    H = 128 if fp8 else 16
    idx = random_routes(rng, T, E, k, mask_prob=0.2)
    w = rng.random((T, k)).astype(np.float32)
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ne = oracle.dispatch_ranked(x, idx, w, E, R, fp8=fp8)
    epr = E // R
    # brute force: rank r's rows are the tokens with an expert on r, ascending
    start = 0
    for r in range(R):
        toks = [t for t in range(T) if any(e >= 0 and e // epr == r for e in idx[t])]
        assert ne["rank_token_offsets"][r] == start
        rows = list(range(start, start + len(toks)))
        assert list(ne["recv_src"][rows]) == toks
        for q, t in zip(rows, toks):
            assert ne["tok_rank_row"][t, r] == q
            for j in range(k):
                e = idx[t, j]
                local = e >= 0 and e // epr == r
                assert ne["recv_topk_idx"][q, j] == (e - r * epr if local else -1)
                assert ne["recv_topk_weights"][q, j] == (w[t, j] if local else 0.0)
        start += len(toks)
    assert ne["rank_token_offsets"][R] == start
    # the receiver's expand is the expanded dispatch of the same route
    ex = oracle.expand(ne, T, k, E, R, A, fp8=fp8)
    d = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8)
    used = int(oracle.layout(idx, E, R, A)["expert_offsets"][-1])
    assert np.array_equal(ex["tok_slot_row"], d["tok_slot_row"])
    for key in ("recv_x", "row_src", "recv_weights") + (("recv_scales",) if fp8 else ()):
        assert np.array_equal(ex[key][:used], d[key][:used]), key


@pytest.mark.parametrize("seed", range(8))
def test_combine_ranked_error_bound(seed):
    rng = np.random.default_rng(5000 + seed)
    T, H, k, E, R = 50, 24, 6, 16, 4
    idx = random_routes(rng, T, E, k, mask_prob=0.1)
    w = rng.random((T, k)).astype(np.float32)
    x = np.zeros((T, H), np.uint16)
    ne = oracle.dispatch_ranked(x, idx, w, E, R)
    d = oracle.dispatch(x, idx, w, E, R)
    cap = T * k
    y = (rng.standard_normal((cap, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out, acc, _ = oracle.combine_ranked(y, d["tok_slot_row"], ne)
    yf = bits_to_f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    mag = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            p = d["tok_slot_row"][t, j]
            if p >= 0:
                exact[t] += np.float64(w[t, j]) * yf[p]
                mag[t] += abs(np.float64(w[t, j])) * np.abs(yf[p])
    assert np.all(np.abs(acc - exact) <= (k + R) * 2.0 ** -24 * mag + 1e-45)
    # and against the single-stage combine: within the combine tolerance
    ref, acc1 = oracle.combine(y, d["tok_slot_row"], w)
    assert np.all(np.abs(acc.astype(np.float64) - acc1) <= 2 * (k + R) * 2.0 ** -24 * mag + 1e-45)


def test_cross_rank_sum_is_in_rank_order():
    """The second stage adds the ranks' fp32 partials in rank order from +0
    (the reading the GPU check is bit-exact against).  Partials 1, 2^24 and
    -2^24 on ranks 0, 1, 2: in rank order 1 + 2^24 rounds to 2^24 (a tie,
    to even) and the sum is 0; in reverse order it would be 1."""
    T, H, k, E, R = 1, 8, 3, 3, 3
    idx = np.array([[0, 1, 2]], np.int32)
    w = np.ones((1, k), np.float32)
    x = np.zeros((T, H), np.uint16)
    ne = oracle.dispatch_ranked(x, idx, w, E, R)
    d = oracle.dispatch(x, idx, w, E, R)
    vals = np.array([1.0, 2.0 ** 24, -(2.0 ** 24)], np.float32)
    y = np.zeros((T * k, H), np.uint16)
    for j in range(k):
        y[d["tok_slot_row"][0, j]] = np.uint16(vals[j:j + 1].view(np.uint32)[0] >> 16)
    out, acc, part = oracle.combine_ranked(y, d["tok_slot_row"], ne)
    assert np.array_equal(part[:, 0], vals)
    assert np.all(acc == 0.0) and np.all(out == 0)


@pytest.mark.parametrize("bits", [0x7F80, 0xFF80, 0x7FC0])
def test_ranked_dispatch_rejects_non_finite_rows(bits):
    """A hidden row holding +inf, -inf or NaN is rejected, as the quantising
    dispatch rejects it ("Deep Dive - DeepEP", "A runnable routing ledger":
    a non-finite row fails the ledger's checks)."""
    x = np.zeros((2, 128), np.uint16)
    x[1, 77] = bits
    idx = np.array([[0, 1], [2, 3]], np.int32)
    for fp8 in (False, True):
        with pytest.raises(oracle.OracleError) as e:
            oracle.dispatch_ranked(x, idx, None, 4, 2, fp8=fp8)
        assert e.value.code == oracle.BAD_ARG
    x[1, 77] = 0x7F7F  # the largest finite bf16 passes
    oracle.dispatch_ranked(x, idx, None, 4, 2)
