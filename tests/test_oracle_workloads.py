"""Oracle invariants on the five synthetic workloads (CPU only).

Tiny: 64 x 128, top-2 of 8 experts on 2 ranks, bf16.
Decode: 128 x 7168, top-8 of 256 on 8 ranks, bf16.
Prefill: 4096 x 7168, top-8 of 256 on 8 ranks, FP8 dispatch.
Skewed: 8192 x 4096, Zipf(1.2) top-6 of 64 on 8 ranks, 5% of slots -1, bf16.
Large: 16384 x 7168, group-limited (4 of 8 groups) top-8 of 256, FP8.
"""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
import ep_workloads as W
from tests.ep_cases import bits_to_f32

NAMES = ["tiny", "decode", "prefill", "skewed", "large"]


@functools.lru_cache(maxsize=8)
def _run(name, with_y):
    w = W.WORKLOADS[name]
    inp = W.generate(w, with_y=with_y)
    lay = oracle.layout(inp["topk_idx"], w.num_experts, w.num_ranks, w.alignment)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_weights"], w.num_experts,
                        w.num_ranks, w.alignment, fp8=w.fp8)
    return w, inp, lay, d


def _renormalised(idx, w):
    """Test-side gates that sum to one over the valid slots (fp64 -> fp32)."""
    w64 = np.where(idx >= 0, w.astype(np.float64), 0.0)
    s = w64.sum(axis=1, keepdims=True)
    s[s == 0] = 1
    return (w64 / s).astype(np.float32)


def test_generator_is_deterministic_and_shaped():
    for name in ("tiny", "decode"):
        w = W.WORKLOADS[name]
        a, b = W.generate(w), W.generate(w)
        for key in a:
            assert np.array_equal(a[key], b[key])
        assert a["x"].shape == (w.num_tokens, w.hidden) and a["x"].dtype == np.uint16
        assert a["topk_idx"].shape == (w.num_tokens, w.num_topk)
        assert a["y"].shape == (w.capacity, w.hidden)
        assert np.allclose(a["topk_weights"].sum(axis=1), 1.0, atol=1e-6)


@pytest.mark.parametrize("name", NAMES)
def test_layout_invariants(name):
    w, inp, lay, d = _run(name, False)
    idx = inp["topk_idx"]
    T, k, E, R = w.num_tokens, w.num_topk, w.num_experts, w.num_ranks
    masked = int((idx < 0).sum())
    if name == "skewed":
        assert masked == math.floor(0.05 * T * k)
    else:
        assert masked == 0
    # distinct experts per token
    s = np.sort(idx, axis=1)
    assert not np.any((s[:, 1:] == s[:, :-1]) & (s[:, 1:] >= 0))
    # counts sum to tokens x top-k minus masked slots
    assert lay["num_tokens_per_expert"].sum() == T * k - masked
    assert lay["expert_offsets"][-1] == T * k - masked  # alignment 1
    # distinct tokens per rank: never more than the rank's expanded rows
    rank_rows = np.diff(lay["rank_offsets"])
    assert np.all(lay["num_tokens_per_rank"] <= rank_rows)
    assert np.array_equal(lay["num_tokens_per_rank"], lay["is_token_in_rank"].sum(axis=0))
    if name == "large":
        assert lay["is_token_in_rank"].sum(axis=1).max() <= w.topk_groups
    if name == "skewed":
        share = (idx == 0).any(axis=1).mean()
        assert 0.8 < share < 0.97  # Zipf(1.2): expert 0 picked by ~90% of tokens


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_expected_destinations_statistically(name):
    """Uniform top-k over E experts on R ranks: distinct destinations per token
    average R * (1 - C(E - E/R, k) / C(E, k)) (5.2947 for 256 / 8 / 8)."""
    w, inp, lay, d = _run(name, False)
    per = lay["is_token_in_rank"].sum(axis=1).astype(np.float64)
    E, R, k = w.num_experts, w.num_ranks, w.num_topk
    closed = R * (1 - math.comb(E - E // R, k) / math.comb(E, k))
    assert abs(per.mean() - closed) <= 4 * per.std() / math.sqrt(len(per)) + 1e-9


@pytest.mark.parametrize("name", NAMES)
def test_dispatch_invariants(name):
    w, inp, lay, d = _run(name, False)
    idx, x = inp["topk_idx"], inp["x"]
    T, k, E = w.num_tokens, w.num_topk, w.num_experts
    tsr, row_src = d["tok_slot_row"], d["row_src"]
    valid = idx >= 0
    assert np.all(tsr[~valid] == -1)
    t_of, j_of = np.nonzero(valid)
    # bijection between valid (t, j) and used rows
    assert np.array_equal(row_src[tsr[t_of, j_of]], t_of * k + j_of)
    used = int(lay["expert_offsets"][-1])
    assert np.all(row_src[:used] >= 0)
    assert len(np.unique(tsr[valid])) == used
    # segments ascending in token order, rows in the right expert segment
    off = lay["expert_offsets"]
    for e in range(E):
        toks = row_src[off[e]:off[e + 1]] // k
        assert np.all(np.diff(toks) > 0)
        assert np.all(idx.reshape(-1)[row_src[off[e]:off[e + 1]]] == e)
    # gates follow their rows
    assert np.array_equal(d["recv_weights"][tsr[t_of, j_of]], inp["topk_weights"][t_of, j_of])
    src_tok = row_src[:used] // k
    if w.fp8:
        # every copy of a token carries the same codes and scales
        first = np.full(T, -1)
        for p in range(used):
            t = src_tok[p]
            if first[t] < 0:
                first[t] = p
        sample = np.arange(0, used, max(1, used // 2000))
        assert np.array_equal(d["recv_x"][sample], d["recv_x"][first[src_tok[sample]]])
        assert np.array_equal(d["recv_scales"][sample], d["recv_scales"][first[src_tok[sample]]])
    else:
        assert np.array_equal(d["recv_x"][:used], x[src_tok])


@pytest.mark.parametrize("name", ["tiny", "decode", "skewed"])
def test_identity_round_trip_bf16(name):
    """Identity experts and gates summing to one: dispatch then combine
    returns x exactly (as values: an input -0 comes back as +0, because the
    fp32 sum starts from +0)."""
    w, inp, lay, d = _run(name, False)
    g = _renormalised(inp["topk_idx"], inp["topk_weights"])
    out, _ = oracle.combine(d["recv_x"], d["tok_slot_row"], g)
    keep = (inp["topk_idx"] >= 0).any(axis=1)
    assert np.array_equal(bits_to_f32(out[keep]), bits_to_f32(inp["x"][keep]))


@pytest.mark.parametrize("name", ["prefill"])
def test_identity_round_trip_fp8(name):
    """FP8 dispatch, a dequantising identity expert, combine: within half an
    e4m3 step (relative 2^-4 for normal codes, 2^-10 * scale for subnormal
    codes) plus two bf16 roundings."""
    w, inp, lay, d = _run(name, False)
    used = int(lay["expert_offsets"][-1])
    q = d["recv_x"][:used]
    s = d["recv_scales"][:used]
    deq = oracle.e4m3_value(q).reshape(used, -1, 128) * s[:, :, None].astype(np.float64)
    y = torch.from_numpy(deq.reshape(used, -1).astype(np.float32)).to(torch.bfloat16)
    y = y.view(torch.int16).numpy().view(np.uint16)
    g = _renormalised(inp["topk_idx"], inp["topk_weights"])
    out, _ = oracle.combine(y, d["tok_slot_row"], g)
    xf = bits_to_f32(inp["x"]).astype(np.float64)
    of = bits_to_f32(out).astype(np.float64)
    T, H = xf.shape
    first = d["tok_slot_row"][:, 0]
    smax = d["recv_scales"][first].astype(np.float64)
    bound = (2.0 ** -4 + 2.0 ** -7) * np.abs(xf) + np.repeat(smax, 128, axis=1) * 2.0 ** -10
    assert np.all(np.abs(of - xf) <= bound)


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_combine_rows_shuffled(name):
    """Combine reads rows only through the handle: permuting the expert rows
    together with the handle leaves the output unchanged."""
    w, _inp, lay, d = _run(name, False)
    inp = W.generate(w, with_y=True)
    used = int(lay["expert_offsets"][-1])
    out, _ = oracle.combine(inp["y"][:used], d["tok_slot_row"], inp["topk_weights"])
    perm = np.random.default_rng(0).permutation(used)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(used)
    tsr = np.where(d["tok_slot_row"] >= 0, inv[np.maximum(d["tok_slot_row"], 0)], -1)
    out2, _ = oracle.combine(inp["y"][:used][perm], tsr.astype(np.int32), inp["topk_weights"])
    assert np.array_equal(out, out2)
