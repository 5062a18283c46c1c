"""Host-side checks of bench.py (CPU only): the algorithmic byte counts and
the scoping of the kernel-source hash that decides whether a stored HBM
counter summary still describes the kernel being timed."""
import bench
import ep_workloads as W

SRC = """// helpers
__device__ int helper(int v) { return v + 1;
}
template <bool kWeighted, int KB>
__global__ __launch_bounds__(kBlock) void combine_kernel(int *p) {
  p[0] = helper(1);
}
template <bool kFp8>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(int *p) {
  p[0] = 2;
}
hipError_t launch_combine(int *p) {
  return hipSuccess;
}
"""


def _h(src, kernel="combine"):
    return bench.kernel_source_hash(kernel, src=src, extra=b"")


def test_hash_ignores_other_kernels():
    assert _h(SRC) == _h(SRC.replace("p[0] = 2;", "p[0] = 3;"))


def test_hash_ignores_comments_and_blank_lines():
    edited = SRC.replace("// helpers", "// helper functions\n\n/* shared */")
    edited = edited.replace("  p[0] = helper(1);", "  p[0] = helper(1);  // the helper")
    assert _h(SRC) == _h(edited)


def test_hash_follows_kernel_launcher_and_helpers():
    base = _h(SRC)
    assert base != _h(SRC.replace("helper(1)", "helper(2)"))
    assert base != _h(SRC.replace("v + 1", "v + 2"))
    assert base != _h(SRC.replace("return hipSuccess;", "return hipErrorUnknown;"))
    assert _h(SRC, "dispatch") != _h(SRC.replace("p[0] = 2;", "p[0] = 3;"), "dispatch")


SRC_USES = """// helpers
__device__ int inner(int v) { return v * 3;
}
__device__ int outer(int v) { return inner(v) + 1;
}
struct Pair {
  int a, b;
};
__device__ int other_only(int v) { return v - 1;
}
constexpr int kUnused = 4;
__device__ int next_to_a_constant(int v) { return v;
}
template <bool kWeighted, int KB>
__global__ __launch_bounds__(kBlock) void combine_kernel(int *p) {
  Pair q{1, 2};
  p[0] = outer(q.a);
}
template <bool kFp8>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(int *p) {
  p[0] = other_only(2);
}
hipError_t launch_combine(int *p) {
  return hipSuccess;
}
"""


def test_hash_follows_only_the_helpers_the_kernel_uses():
    base = _h(SRC_USES)
    # used directly, through another helper, or as a type
    assert base != _h(SRC_USES.replace("inner(v) + 1", "inner(v) + 2"))
    assert base != _h(SRC_USES.replace("v * 3", "v * 4"))
    assert base != _h(SRC_USES.replace("int a, b;", "int a, b, c;"))
    # used by another kernel only
    assert base == _h(SRC_USES.replace("v - 1", "v - 2"))
    assert _h(SRC_USES, "dispatch") != _h(SRC_USES.replace("v - 1", "v - 2"), "dispatch")
    # a piece holding more than one definition is always taken
    assert base != _h(SRC_USES.replace("kUnused = 4", "kUnused = 5"))


def test_measured_kernels_take_their_helpers_from_the_real_source():
    with open(bench.KERNEL_SOURCES[0]) as f:
        src = f.read()
    names = {bench._sole_definition(p) for p in bench.split_functions(src)
             if bench._piece_name(p)[0] == "helper"}
    # helpers of each measured kernel are recognised as single definitions
    for helper in ("gather_rows", "quantize16", "load_x_slice", "count_tile", "scan_counts",
                   "launch_kernel"):
        assert helper in names

    def edited(helper, kernel):
        pieces = bench.split_functions(src)
        for i, p in enumerate(pieces):
            if bench._piece_name(p)[0] == "helper" and bench._sole_definition(p) == helper:
                body = p.rstrip()
                pieces[i] = body[:-1] + "  (void)0;\n}\n"
        return bench.kernel_source_hash(kernel, src="".join(pieces), extra=b"")

    def plain(kernel):
        return bench.kernel_source_hash(kernel, src=src, extra=b"")

    assert edited("gather_rows", "combine") != plain("combine")
    assert edited("quantize16", "dispatch") != plain("dispatch")
    assert edited("count_tile", "layout") != plain("layout")
    assert edited("quantize16", "combine") == plain("combine")
    assert edited("gather_rows", "layout") == plain("layout")


def test_every_measured_kernel_is_found_in_the_source():
    with open(bench.KERNEL_SOURCES[0]) as f:
        src = f.read()
    pieces = bench.split_functions(src)
    assert "".join(pieces) == src
    names = {bench._piece_name(p)[1] for p in pieces}
    for kname, lname in bench.KERNEL_FUNCS.values():
        assert kname in names and lname in names


def test_algorithmic_bytes_prefill_closed_form():
    """Prefill: 4096 x 7168, top-8, E=256, R=8, FP8 rows of H + H/32 bytes,
    every selection valid (M = T*k)."""
    w = W.WORKLOADS["prefill"]
    T, H, k, E, R = 4096, 7168, 8, 256, 8
    M = T * k
    by = bench.algorithmic_bytes(w, M)
    assert by["layout"] == T * k * 4 + T * R + 4 * (E + R) + 4 * (E + R + 2) == 165960
    assert by["dispatch"] == T * H * 2 + T * k * 12 + M * (H + H // 32 + 8) == 301596672
    assert by["combine"] == M * 2 * H + T * k * 8 + T * 2 * H == 528744448


def test_short_kernel_name_keeps_anonymous_namespace_kernels():
    """Profiler names lose their argument list but never their identity."""
    assert bench.short_kernel_name(
        "void ep::combine_kernel<true, 8>(ep::Dims, int, long)") == "ep::combine_kernel<true, 8>"
    assert bench.short_kernel_name(
        "void (anonymous namespace)::probe_copy<true>(unsigned int __vector(4) const*, long)"
    ) == "anon::probe_copy<true>"
    assert bench.short_kernel_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def _oracle_step(w):
    import oracle

    inp = W.generate(w)
    lay = oracle.layout(inp["topk_idx"], w.num_experts, w.num_ranks, w.alignment)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_weights"], w.num_experts,
                        w.num_ranks, w.alignment, fp8=w.fp8)
    out, _ = oracle.combine(inp["y"], d["tok_slot_row"], inp["topk_weights"])
    rows = int(lay["expert_offsets"][-1])
    got = {n: lay[n].copy() for n in ("num_tokens_per_rank", "num_tokens_per_expert",
                                      "is_token_in_rank", "expert_offsets", "rank_offsets")}
    got["tok_slot_row"] = d["tok_slot_row"].copy()
    for n in ("row_src", "recv_weights", "recv_x"):
        got[n] = d[n][:rows].copy()
    got["recv_scales"] = None if d["recv_scales"] is None else d["recv_scales"][:rows].copy()
    got["out"] = out.copy()
    return got, lay, d, out


def test_step_comparison_flags_each_part():
    """The bench's check of the timed step against the oracle: equal outputs
    pass, and one changed value in any part fails that part only."""
    import dataclasses

    for w in (W.WORKLOADS["tiny"], dataclasses.replace(W.WORKLOADS["tiny"], fp8=True)):
        got, lay, d, out = _oracle_step(w)
        assert bench.compare_step(got, lay, d, out) == {
            "layout": True, "handle": True, "rows": True, "combine_bits": True, "all": True}
        cases = [("expert_offsets", "layout"), ("row_src", "handle"),
                 ("recv_weights", "handle"), ("recv_x", "rows"), ("out", "combine_bits")]
        if w.fp8:
            cases.append(("recv_scales", "rows"))
        for name, part in cases:
            bad = dict(got)
            arr = got[name].copy()
            flat = arr.reshape(-1)
            flat[flat.size // 2] = flat[flat.size // 2] + 1
            bad[name] = arr
            res = bench.compare_step(bad, lay, d, out)
            assert not res[part] and not res["all"], (name, res)
            assert all(v for k, v in res.items() if k not in (part, "all")), (name, res)


def test_logical_network_bytes_counts_token_rank_rows():
    """One row per (token, destination rank), counted from a layout the
    oracle wrote for a hand-checked route: 6 rows for 8 assignments."""
    import types

    import numpy as np
    import torch

    import oracle

    # tokens 0..3, 4 experts on 2 ranks (experts 0,1 on rank 0; 2,3 on rank 1)
    idx = np.array([[0, 1], [0, 2], [2, 3], [1, 3]], np.int32)
    lay = oracle.layout(idx, 4, 2, 1)
    b = types.SimpleNamespace(
        is_token_in_rank=torch.from_numpy(lay["is_token_in_rank"]),
        num_tokens_per_expert=torch.from_numpy(lay["num_tokens_per_expert"]))
    w = types.SimpleNamespace(num_tokens=4, hidden=256, num_ranks=2, fp8=False)
    got = bench.logical_network_bytes(w, b)
    # rows: token 0 -> {0}, 1 -> {0, 1}, 2 -> {1}, 3 -> {0, 1}: 6 rows
    assert got["rows"] == 6 and got["expanded_rows_per_token"] == 2.0
    assert got["dispatch_bytes"] == 6 * 512 and got["combine_bytes"] == 6 * 512
    # owners t*R/T: tokens 0, 1 on rank 0, tokens 2, 3 on rank 1; remote rows:
    # token 1 -> rank 1, token 3 -> rank 0
    assert got["remote_rows"] == 2
    w8 = types.SimpleNamespace(num_tokens=4, hidden=256, num_ranks=2, fp8=True)
    assert bench.logical_network_bytes(w8, b)["dispatch_bytes"] == 6 * (256 + 8)


def test_mode_trace_summary_lists_every_kernel(tmp_path, monkeypatch):
    """The summary of a --ranked or backward trace keeps each kernel's calls
    and its average, minimum and maximum duration, in microseconds."""
    run = tmp_path / "run" / "trace"
    run.mkdir(parents=True)
    (run / "ep_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void ep::expand_kernel<true>(ep::Dims, int)",3,300000,100000,50.0,90000,110000,1.0\n'
        '"__amd_rocclr_copyBuffer",2,5000,2500,1.0,2000,3000,1.0\n')
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(root))
    bench.mode_trace_summary(str(tmp_path / "run"), "ranked", "non-expanded path", "prefill",
                             "rocprofv3 ... -- python3 bench.py --ranked")
    text = (root / "profiles" / "ranked_prefill_kernel_trace.md").read_text()
    assert "python3 bench.py --ranked" in text
    assert "| ep::expand_kernel<true> | 3 | 100.00 | 90.00 | 110.00 |" in text
    assert "| __amd_rocclr_copyBuffer | 2 | 2.50 | 2.00 | 3.00 |" in text
