"""Mutation check of the oracle's pins (CPU only; not collected by pytest).

Each mutation plants one typical mistake in a copy of oracle/oracle.c: a
dropped or wrong rounding step, a reversed order, a wrong index, scale,
weight, rank or padding value.  The copy is built with the oracle's own gcc
flags and the oracle tests are run against it (the oracle loader takes the
build named by EP_ORACLE_LIB).  A mutation is "caught" when at least one
test fails.  Every mutation must be caught: a surviving one names an
arithmetic step of the oracle that no pin fixes.

    python tests/oracle_mutations.py            # all mutations, 4 at a time
    python tests/oracle_mutations.py -k fp8     # those whose name contains fp8

Exit status 0 when every selected mutation is caught.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
HDR = os.path.join(ROOT, "oracle", "oracle.h")
TESTS = ["tests/test_oracle_readings.py", "tests/test_oracle_pins.py",
         "tests/test_oracle_ranked.py", "tests/test_oracle_backward.py",
         "tests/test_oracle_workloads.py"]

# (name, text in oracle.c, replacement, which occurrence of the text (0 = first))
MUTATIONS = [
    # bf16 rounding ("Deep Dive - DeepEP", "Combine: reverse routing plus reduction")
    ("bf16_ties_away", "bits + 0x7FFFu + lsb", "bits + 0x8000u", 0),
    ("bf16_ties_down", "bits + 0x7FFFu + lsb", "bits + 0x7FFFu", 0),
    # E4M3 encoding
    ("e4m3_ties_up", "code = (lo % 2 == 0) ? lo : hi;", "code = hi;", 0),
    ("e4m3_saturate_to_nan", "return sign | 0x7E;", "return sign | 0x7F;", 0),
    ("e4m3_unsigned_zero", "uint8_t sign = signbit(v) ? 0x80 : 0x00;",
     "uint8_t sign = (v < 0) ? 0x80 : 0x00;", 0),
    ("e4m3_no_subnormals", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);", 0),
    # FP8 block quantiser ("Precision: FP8 on the wire, BF16 for the reduction")
    ("fp8_scale_by_reciprocal", "float scale = amax / 448.0f;",
     "float scale = amax * (1.0f / 448.0f);", 0),
    ("fp8_codes_by_multiplier", "float v = oracle_bf16_to_float(xrow[b * 128 + c]) / scale;",
     "float v = oracle_bf16_to_float(xrow[b * 128 + c]) * (448.0f / amax);", 0),
    ("fp8_scale_240", "float scale = amax / 448.0f;", "float scale = amax / 240.0f;", 0),
    ("fp8_amax_half_block", "for (int c = 0; c < 128; ++c) {\n      float v = fabsf",
     "for (int c = 0; c < 64; ++c) {\n      float v = fabsf", 0),
    ("fp8_zero_block_code", "q[b * 128 + c] = 0x00;", "q[b * 128 + c] = 0x80;", 0),
    # validation
    ("route_repeats_allowed", "if (idx[t * k + jj] == e) return ORACLE_BAD_ROUTE;",
     "if (0) return ORACLE_BAD_ROUTE;", 0),
    ("nonfinite_allowed",
     "if (!isfinite(oracle_bf16_to_float(x[i]))) return ORACLE_BAD_ARG;",
     "if (0) return ORACLE_BAD_ARG;", 0),
    ("gates_nonfinite_allowed",
     "if (idx[t * k + j] >= 0 && !isfinite(w[t * k + j])) return ORACLE_BAD_ARG;",
     "if (0) return ORACLE_BAD_ARG;", 0),
    ("gates_checked_on_unused_slots",
     "if (idx[t * k + j] >= 0 && !isfinite(w[t * k + j])) return ORACLE_BAD_ARG;",
     "if (!isfinite(w[t * k + j])) return ORACLE_BAD_ARG;", 0),
    # layout ("6.1 Layout Metadata", "Dispatch: layout, move, and epilogue")
    ("count_skips_expert0", "if (e >= 0) num_tokens_per_expert[e] += 1;",
     "if (e > 0) num_tokens_per_expert[e] += 1;", 0),
    ("rank_by_modulo", "is_token_in_rank[t * R + e / experts_per_rank] = 1;",
     "is_token_in_rank[t * R + e % R] = 1;", 0),
    ("align_overpads", "((int64_t)num_tokens_per_expert[e] + A - 1) / A * A",
     "((int64_t)num_tokens_per_expert[e] + A) / A * A", 0),
    ("rank_offsets_by_rank", "rank_offsets[r] = expert_offsets[r * experts_per_rank];",
     "rank_offsets[r] = expert_offsets[r];", 0),
    # dispatch placement and handle ("7.1 Does Sort Exist?", ledger)
    ("segment_descending", "int64_t p = off[e] + fill[e];",
     "int64_t p = off[e] + cnt[e] - 1 - fill[e];", 0),
    ("row_src_token_only", "row_src[p] = (int32_t)(t * k + j);", "row_src[p] = (int32_t)t;", 0),
    ("recv_weight_slot0", "if (recv_weights && topk_weights) recv_weights[p] = topk_weights[t * k + j];",
     "if (recv_weights && topk_weights) recv_weights[p] = topk_weights[t * k];", 0),
    ("padding_weight_one", "if (recv_weights && topk_weights) recv_weights[p] = 0.0f;",
     "if (recv_weights && topk_weights) recv_weights[p] = 1.0f;", 0),
    ("padding_source_zero", "row_src[p] = -1;", "row_src[p] = 0;", 0),
    ("fp8_input_scale_of_token0",
     "memcpy(recv_scales + p * nblk, x_scales + t * nblk, sizeof(float) * (size_t)nblk);",
     "memcpy(recv_scales + p * nblk, x_scales, sizeof(float) * (size_t)nblk);", 0),
    # combine ("Combine: reverse routing plus reduction")
    ("combine_gate_of_slot0", "acc = fmaf(topk_weights[t * k + j], yv, acc);",
     "acc = fmaf(topk_weights[t * k], yv, acc);", 0),
    ("combine_reversed_order",
     "for (int j = 0; j < k; ++j) {\n        int64_t p = tok_slot_row[t * k + j];\n"
     "        if (p < 0) continue;\n        float yv",
     "for (int j = k - 1; j >= 0; --j) {\n        int64_t p = tok_slot_row[t * k + j];\n"
     "        if (p < 0) continue;\n        float yv", 0),
    ("combine_mul_then_add", "acc = fmaf(topk_weights[t * k + j], yv, acc);",
     "acc = acc + topk_weights[t * k + j] * yv;", 0),
    ("combine_truncates", "out[t * H + c] = oracle_bf16_round(acc);",
     "out[t * H + c] = (uint16_t)(f32_bits(acc) >> 16);", 0),
    ("combine_starts_negative_zero", "float acc = 0.0f;\n      for (int j = 0; j < k; ++j) {\n"
     "        int64_t p = tok_slot_row[t * k + j];\n        if (p < 0) continue;\n        float yv",
     "float acc = -0.0f;\n      for (int j = 0; j < k; ++j) {\n"
     "        int64_t p = tok_slot_row[t * k + j];\n        if (p < 0) continue;\n        float yv", 0),
    # non-expanded path ("Why expert parallelism needs a communication layer")
    ("ranked_rank_by_modulo", "if (e >= 0 && e / epr == r) in = 1;",
     "if (e >= 0 && e % R == r) in = 1;", 0),
    ("ranked_global_expert_id", "recv_topk_idx[q * k + j] = local ? e - r * epr : -1;",
     "recv_topk_idx[q * k + j] = local ? e : -1;", 0),
    ("ranked_weights_not_local",
     "(local && topk_weights) ? topk_weights[t * k + j] : 0.0f",
     "topk_weights ? topk_weights[t * k + j] : 0.0f", 0),
    ("ranked_nonfinite_allowed",
     "if (!isfinite(oracle_bf16_to_float(x[i]))) return ORACLE_BAD_ARG;",
     "if (0) return ORACLE_BAD_ARG;", 1),
    ("expand_weight_one", "if (recv_weights && recv_topk_weights) recv_weights[p] = recv_topk_weights[q * k + j];",
     "if (recv_weights && recv_topk_weights) recv_weights[p] = 1.0f;", 0),
    ("expand_row_src_token_only", "row_src[p] = (int32_t)(t * k + j);", "row_src[p] = (int32_t)t;", 2),
    ("ranked_stage1_reversed",
     "for (int j = 0; j < k; ++j) {\n        if (recv_topk_idx[q * k + j] < 0) continue;",
     "for (int j = k - 1; j >= 0; --j) {\n        if (recv_topk_idx[q * k + j] < 0) continue;", 0),
    ("ranked_stage1_mul_then_add", "acc = fmaf(recv_topk_weights[q * k + j], yv, acc);",
     "acc = acc + recv_topk_weights[q * k + j] * yv;", 0),
    ("ranked_stage2_reversed", "for (int r = 0; r < R; ++r) {\n        int64_t q = tok_rank_row",
     "for (int r = R - 1; r >= 0; --r) {\n        int64_t q = tok_rank_row", 0),
    ("ranked_bf16_partials", "part[q * H + c] = acc;",
     "part[q * H + c] = oracle_bf16_to_float(oracle_bf16_round(acc));", 0),
    # backward ("Combine: reverse routing plus reduction", backward duality)
    ("dispatch_backward_reversed",
     "for (int j = 0; j < k; ++j) {\n        int64_t p = tok_slot_row[t * k + j];\n"
     "        if (p < 0) continue;\n        acc = acc + oracle_bf16_to_float(grad_recv",
     "for (int j = k - 1; j >= 0; --j) {\n        int64_t p = tok_slot_row[t * k + j];\n"
     "        if (p < 0) continue;\n        acc = acc + oracle_bf16_to_float(grad_recv", 0),
    ("dispatch_backward_truncates", "grad_x[t * H + c] = oracle_bf16_round(acc);",
     "grad_x[t * H + c] = (uint16_t)(f32_bits(acc) >> 16);", 0),
    ("combine_backward_no_gate", "grad_expert_out[p * H + c] = oracle_bf16_round(w * g);",
     "grad_expert_out[p * H + c] = oracle_bf16_round(g);", 0),
    ("gate_gradient_weighted",
     "double term = (double)oracle_bf16_to_float(expert_out[p * H + c]) * (double)g;",
     "double term = (double)oracle_bf16_to_float(expert_out[p * H + c]) * (double)g * (double)w;", 0),
    ("backward_padding_not_zeroed",
     "for (int64_t i = 0; i < rows_used * H; ++i) grad_expert_out[i] = 0;",
     "for (int64_t i = 0; i < 0; ++i) grad_expert_out[i] = 0;", 0),
]

def mutate(src: str, old: str, new: str, nth: int) -> str:
    pos = -1
    for _ in range(nth + 1):
        pos = src.find(old, pos + 1)
        if pos < 0:
            raise SystemExit(f"mutation text not found (occurrence {nth}): {old!r}")
    return src[:pos] + new + src[pos + len(old):]


def run_one(m, gcc_flags, tmp_root, verbose):
    name, old, new, nth = m
    with open(SRC) as f:
        src = f.read()
    d = tempfile.mkdtemp(prefix=f"mut_{name}_", dir=tmp_root)
    shutil.copy(HDR, d)
    with open(os.path.join(d, "oracle.c"), "w") as f:
        f.write(mutate(src, old, new, nth))
    lib = os.path.join(d, "liboracle.so")
    b = subprocess.run(["gcc", *gcc_flags, os.path.join(d, "oracle.c"), "-o", lib, "-lm"],
                       capture_output=True, text=True)
    if b.returncode != 0:
        return name, "build failed", b.stderr[-2000:]
    env = dict(os.environ, EP_ORACLE_LIB=lib)
    t0 = time.perf_counter()
    r = subprocess.run([sys.executable, "-m", "pytest", *TESTS, "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    el = time.perf_counter() - t0
    first = next((l for l in r.stdout.splitlines() if l.startswith("FAILED")), "")
    if r.returncode == 0:
        return name, "SURVIVED", f"({el:.0f} s)"
    if r.returncode != 1:
        return name, f"caught (pytest exit {r.returncode})", f"({el:.0f} s) " + first
    return name, "caught", f"({el:.0f} s) " + (first if verbose else first[:110])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("-k", default="", help="only mutations whose name contains this")
    ap.add_argument("-j", type=int, default=4, help="mutations run at once")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    import oracle

    flags = [f for f in oracle.GCC_FLAGS]
    sel = [m for m in MUTATIONS if args.k in m[0]]
    # a mutation must change the source, and its text must be present
    with open(SRC) as f:
        src = f.read()
    for m in sel:
        assert m[1] != m[2], m[0]
        mutate(src, m[1], m[2], m[3])
    tmp_root = tempfile.mkdtemp(prefix="oracle_mutations_")
    survived = 0
    try:
        with cf.ThreadPoolExecutor(args.j) as ex:
            for name, verdict, detail in ex.map(lambda m: run_one(m, flags, tmp_root, args.v),
                                                sel):
                print(f"{name:32s} {verdict:10s} {detail}", flush=True)
                survived += verdict != "caught" and not verdict.startswith("caught")
    finally:
        shutil.rmtree(tmp_root, ignore_errors=True)
    print(f"{len(sel) - survived} of {len(sel)} mutations caught")
    sys.exit(1 if survived else 0)


if __name__ == "__main__":
    main()
