"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact for counts, offsets, rank mask, permutation (tok_slot_row),
source indices (row_src), received gates, bf16 rows, FP8 codes and scales;
combine within 2^-7 relative of the oracle's fp32 accumulator (plus a
cancellation allowance of k * 2^-24 * sum |w y|), and in practice bit-equal
to the oracle's bf16 output because both use the same slot order and fused
multiply-adds.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import combine_get_dispatch_amd as ep  # noqa: E402
import ep_workloads as W  # noqa: E402
import oracle  # noqa: E402
from tests.ep_cases import Ledger, bf16_bits_exact, bits_to_f32, row_experts  # noqa: E402
from tests.gpu_backend import GpuBackend, dev, dev_bf16, host_bf16, say  # noqa: E402

GPU = GpuBackend()


def combine_tolerance_ok(got_bits, ref_bits, acc, y_bits, tsr, w):
    """Per element: bit-equal to the oracle's bf16, or within 2^-7 relative of
    the oracle's fp32 accumulator plus k * 2^-24 * sum_j |w_j y_j|."""
    got = bits_to_f32(got_bits).astype(np.float64)
    a = acc.astype(np.float64)
    same = got_bits == ref_bits
    if same.all():
        return True, 0
    T, k = tsr.shape
    mag = np.zeros_like(a)
    yf = bits_to_f32(y_bits)
    for j in range(k):
        r = tsr[:, j]
        ok = r >= 0
        wj = np.ones(T) if w is None else np.abs(w[:, j].astype(np.float64))
        mag[ok] += wj[ok, None] * np.abs(yf[r[ok]].astype(np.float64))
    bound = 2.0 ** -7 * np.abs(a) + k * 2.0 ** -24 * mag
    within = same | (np.abs(got - a) <= bound)
    return bool(within.all()), int((~same).sum())


def run_gpu_workload(w, inp):
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    say(f"workload {w.name}: T={T} H={H} k={k} E={w.num_experts} R={w.num_ranks} fp8={w.fp8}")
    b = ep.EpBuffers(T, H, k, w.num_experts, w.num_ranks, w.alignment, fp8=w.fp8)
    b.row_src.fill_(-2)
    idx = dev(inp["topk_idx"])
    wts = dev(inp["topk_weights"])
    x = dev_bf16(inp["x"])
    y = dev_bf16(inp["y"])
    rows = b.layout(idx, sync=True)
    b.dispatch(x, idx, wts)
    out = b.combine(y, wts)
    b.check_status()
    torch.cuda.synchronize()
    return b, rows, out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "large"])
def test_workload_parity(name):
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    b, rows, out = run_gpu_workload(w, inp)
    lay = oracle.layout(inp["topk_idx"], w.num_experts, w.num_ranks, w.alignment)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_weights"], w.num_experts,
                        w.num_ranks, w.alignment, fp8=w.fp8)
    used = int(lay["expert_offsets"][-1])
    assert rows == used
    for key in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
                "expert_offsets", "rank_offsets"):
        assert np.array_equal(getattr(b, key).cpu().numpy(), lay[key]), key
    assert np.array_equal(b.tok_slot_row.cpu().numpy(), d["tok_slot_row"])
    assert np.array_equal(b.row_src[:used].cpu().numpy(), d["row_src"][:used])
    assert np.array_equal(b.recv_weights[:used].cpu().numpy().view(np.uint32),
                          d["recv_weights"][:used].view(np.uint32))
    if w.fp8:
        assert np.array_equal(b.recv_x[:used].cpu().numpy(), d["recv_x"][:used])
        assert np.array_equal(b.recv_scales[:used].cpu().numpy().view(np.uint32),
                              d["recv_scales"][:used].view(np.uint32))
    else:
        assert np.array_equal(host_bf16(b.recv_x[:used]), d["recv_x"][:used])
    ref, acc = oracle.combine(inp["y"], d["tok_slot_row"], inp["topk_weights"])
    got = host_bf16(out)
    ok, ndiff = combine_tolerance_ok(got, ref, acc, inp["y"], d["tok_slot_row"],
                                     inp["topk_weights"])
    assert ok, f"{ndiff} elements outside tolerance"
    assert ndiff == 0, f"{ndiff} elements within tolerance but not bit-equal"


# --------------------------------------------------------------------------
# the pages' worked examples, replayed on the GPU
# --------------------------------------------------------------------------

class OracleBackend:
    hidden_multiple = 8

    def layout(self, idx, E, R, A):
        return oracle.layout(idx, E, R, A)

    def dispatch(self, x, idx, w, E, R, A, fp8, cap):
        return oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=cap)

    def combine(self, y, tsr, w):
        return oracle.combine(y, tsr, w)[0]


ORC = OracleBackend()


@pytest.mark.parametrize("alignment", [1, 4])
@pytest.mark.parametrize("weighting", ["combine", "caller", "none", "twice"])
def test_ledger_on_gpu(alignment, weighting):
    L = Ledger()
    idx, w = L.routes()
    g = L.run(GPU, idx, w, alignment, weighting)
    o = L.run(ORC, idx, w, alignment, weighting)
    assert np.array_equal(g["out"], o["out"])
    assert g["rows_used"] == o["rows_used"]
    for key in ("tok_slot_row", "row_src", "recv_weights", "recv_x"):
        assert np.array_equal(g["dispatch"][key][: g["rows_used"]] if key != "tok_slot_row"
                              else g["dispatch"][key],
                              o["dispatch"][key][: o["rows_used"]] if key != "tok_slot_row"
                              else o["dispatch"][key]), key
    if weighting == "combine":
        for i, t in enumerate(L.tokens):
            want = np.array(L.fx.nums(f"expect.{t}"))
            assert np.all(np.abs(g["out"][i] - want) <= 0.005 + 2.0 ** -7 * np.abs(want))


def test_ledger_variants_on_gpu():
    L = Ledger()
    v = L.var
    idx, w = L.routes({"a": v["same_rank.route.a"]})
    g = L.run(GPU, idx, w)
    assert g["layout"]["num_tokens_per_rank"].sum() == v.num("same_rank.destination_rows", int)
    assert g["layout"]["num_tokens_per_expert"].sum() == v.num("same_rank.assignments", int)
    assert abs(g["out"][0, 0] - v.num("same_rank.expect.a0")) <= 0.005 + 2.0 ** -7 * 3.3
    idx, w = L.routes({"a": v["masked.route.a"]})
    w[0, 1] = np.nan  # never read
    g = L.run(GPU, idx, w)
    o = L.run(ORC, idx, w)
    assert np.array_equal(g["out"], o["out"])
    assert g["layout"]["num_tokens_per_rank"].sum() == v.num("masked.destination_rows", int)


def test_t0_and_fragment_and_alignment_on_gpu(golden):
    fx = golden("t0_example.txt")
    idx = np.array([fx.nums(f"route.{t}", int) for t in ("T0", "T1", "T2")], np.int32)
    lay = GPU.layout(idx, fx.num("num_experts", int), fx.num("num_ranks", int), 1)
    assert list(lay["num_tokens_per_expert"]) == fx.nums("counts", int)
    assert list(lay["expert_offsets"]) == fx.nums("offsets", int)
    assert list(lay["num_tokens_per_rank"]) == fx.nums("distinct_tokens_per_rank", int)
    fr = golden("layout_fragment.txt")
    idx = np.array([[2]] * fr.num("expert2_count", int) + [[3]] * fr.num("expert3_count", int),
                   np.int32)
    lay = GPU.layout(idx, 4, 1, 1)
    assert lay["expert_offsets"][2] == fr.num("expert2_offset", int)
    assert lay["expert_offsets"][3] == fr.num("expert3_offset", int)
    al = golden("alignment.txt")
    c = al.nums("counts", int)
    idx = np.array([[0]] * c[0] + [[1]] * c[1], np.int32)
    lay = GPU.layout(idx, 2, 1, al.num("alignment", int))
    assert list(lay["expert_offsets"][:2]) == al.nums("starts", int)
    assert list(lay["expert_offsets"][:2] + lay["num_tokens_per_expert"]) == al.nums("ends", int)
    assert lay["expert_offsets"][2] == al.num("total_slots", int)


def test_cancellation_on_gpu(golden):
    fx = golden("cancellation.txt")
    c = fx.nums("contributions")
    y = bf16_bits_exact(np.array(c, np.float32)[:, None] * np.ones((1, 8), np.float32))
    tsr = np.array([[0, 1, 2]], np.int32)
    assert np.all(bits_to_f32(GPU.combine(y, tsr, None)) == fx.num("fp32_sum_then_bf16"))
    assert np.all(bits_to_f32(GPU.combine(y, tsr, np.ones((1, 3), np.float32)))
                  == fx.num("fp32_sum_then_bf16"))


# --------------------------------------------------------------------------
# random small shapes: ragged tiles and chunks, masks, alignment, dtypes
# --------------------------------------------------------------------------

def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    fp8 = bool(seed % 3 == 0)
    T = int(rng.choice([1, 5, 63, 64, 65, 255, 256, 257, 300, 700, 1000]))
    H = int(rng.choice([128, 384, 1152, 2048]) if fp8 else rng.choice([8, 24, 136, 520, 1032, 2056]))
    R = int(rng.choice([1, 2, 4, 8]))
    E = R * int(rng.integers(1, 9))
    k = int(rng.integers(1, min(E, 9) + 1))
    A = int(rng.choice([1, 1, 2, 4, 16]))
    idx = W.random_routes(rng, T, E, k, mask_prob=float(rng.choice([0.0, 0.1, 0.5])))
    x = W.normal_bf16(rng, (T, H), float(rng.choice([1.0, 1e-3, 30.0])))
    w = rng.random((T, k)).astype(np.float32)
    cap = T * k + E * (A - 1)
    y = W.normal_bf16(rng, (cap, H))
    return fp8, T, H, k, E, R, A, idx, x, w, cap, y


@pytest.mark.parametrize("seed", range(36))
def test_random_small_parity(seed):
    fp8, T, H, k, E, R, A, idx, x, w, cap, y = _random_case(seed)
    lg = GPU.layout(idx, E, R, A)
    lo = oracle.layout(idx, E, R, A)
    for key in lo:
        assert np.array_equal(lg[key], lo[key]), key
    dg = GPU.dispatch(x, idx, w, E, R, A, fp8, cap)
    do = oracle.dispatch(x, idx, w, E, R, A, fp8=fp8, capacity=cap)
    used = int(lo["expert_offsets"][-1])
    assert np.array_equal(dg["tok_slot_row"], do["tok_slot_row"])
    for key in ("row_src", "recv_x", "recv_weights") + (("recv_scales",) if fp8 else ()):
        assert np.array_equal(dg[key][:used], do[key][:used]), key
    og = GPU.combine(y, do["tok_slot_row"], w)
    oo, acc = oracle.combine(y, do["tok_slot_row"], w)
    assert np.array_equal(og, oo)
    og = GPU.combine(y, do["tok_slot_row"], None)
    oo, _ = oracle.combine(y, do["tok_slot_row"], None)
    assert np.array_equal(og, oo)
