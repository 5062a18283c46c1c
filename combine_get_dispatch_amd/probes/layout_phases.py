"""Phase timestamps of the layout kernel: a measurement aid, not on the path.

Writes an instrumented copy of csrc/ep_kernels.hip to a temporary directory.
Thread 0 of every layout workgroup reads the 100 MHz real-time counter
(s_memrealtime) at the end of each phase into LDS and writes the record out
as the workgroup exits, so that the probe adds no memory operation inside the
phases (the ids-loaded mark alone forces a wait for the ids, which the real
kernel overlaps with its LDS clear).  A small harness then launches the
layout through the library's own launcher on synthetic routes (uniform,
distinct top-k) and prints, per batch, the median over 40 launches of:

  - each phase's end, in microseconds from the first workgroup's start: the
    latest over the workgroups for the shared phases, the scanning
    workgroup's own for the scan phases;
  - the kernel's time between its start and stop events.

Each launch follows an idle GPU (a synchronisation and a copy), so the
figures hold a cold-start cost that back-to-back launches hide; compare
variants with each other, not with a trace.

    python combine_get_dispatch_amd/probes/layout_phases.py [--shapes T:k:E:R,...]

Needs hipcc and, to run, the GPU.  The anchors are exact source lines of the
layout kernel: when the kernel changes, the script stops and names the
anchor it could not find.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
sys.path.insert(0, ROOT)
from combine_get_dispatch_amd import _build  # noqa: E402

PHASES = [  # (slot, label, whose figure)
    (0, "last workgroup starts", "all"),
    (1, "ids loaded", "all"),
    (2, "masks cleared", "all"),
    (3, "marking issued", "all"),
    (4, "rank ballots, barrier", "all"),
    (5, "count done", "all"),
    (6, "row published (release)", "all"),
    (7, "ticket drawn", "all"),
    (11, "other workgroups' outputs issued", "all"),
    (13, "scanner: acquired", "scanner"),
    (12, "scanner: loads issued", "scanner"),
    (8, "scanner: totals ready", "scanner"),
    (9, "scanner: scan done", "scanner"),
    (10, "scanner: last store issued", "scanner"),
]


def _mark(i: int) -> str:
    return f"\n  if (threadIdx.x == 0) s_ts[{i}] = __builtin_amdgcn_s_memrealtime();\n"


def _insert(text: str, anchor: str, slot: int, after: bool = True) -> str:
    if text.count(anchor) != 1:
        raise SystemExit(f"layout_phases: anchor for phase {slot} found {text.count(anchor)} "
                         f"times (expected once):\n{anchor}")
    p = text.index(anchor) + (len(anchor) if after else 0)
    return text[:p] + _mark(slot) + text[p:]


def instrument(src: str) -> str:
    a = src.index("__device__ __forceinline__ void count_tile(")
    b = src.index("// Stable rank of selection e")
    c = src[a:b]
    c = _insert(c, "  for (int i = tid; i < R; i += kBlock) L.rank_cnt[i] = 0;\n"
                   "  __syncthreads();\n", 2)
    c = _insert(c, "  // A repeated expert within the token is checked", 3, after=False)
    c = _insert(c, "    if (mine) atomicAdd(&L.rank_cnt[lane], (int32_t)__popcll(mine));\n"
                   "  }\n  __syncthreads();\n", 4)
    src = src[:a] + c + src[b:]

    a = src.index("__global__ __launch_bounds__(kBlock) void layout_kernel(")
    b = src.index("// Zeroes the workspace header")
    k = src[a:b]
    k = k.replace("  int32_t ex[K];\n", "  int32_t ex[K];\n  if (threadIdx.x == 0)\n"
                  "    for (int q_ = 1; q_ < 16; ++q_) s_ts[q_] = 0;\n", 1)
    k = _insert(k, "  int32_t ex[K];\n", 0)
    wait = '    asm volatile("" :: "v"(ex[0]), "v"(ex[K - 1]));\n'
    k = k.replace("    load_ids<K>(d, t, live, topk_idx, ex);\n",
                  "    load_ids<K>(d, t, live, topk_idx, ex);\n" + wait, 1)
    k = _insert(k, wait, 1)
    k = _insert(k, "    count_tile<K>(d, tile, experts_per_rank, L, ex, rmask, rank_ballot_ws, "
                   "status);\n", 5)
    k = _insert(k, '      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");\n', 6)
    k = _insert(k, "  const bool scans = !many || is_last;\n", 7)
    exit_other = ("  if (!scans) {\n    if (live) token_outputs<K>(d, t, L, ex, rmask, "
                  "is_token_in_rank, slot_rank);\n    return;\n  }\n")
    if k.count(exit_other) != 1:
        raise SystemExit("layout_phases: the non-scanning workgroups' exit changed")
    k = k.replace(exit_other, exit_other.replace("    return;\n", _mark(11) + "    FLUSH;\n"
                                                 "    return;\n"))
    k = _insert(k, '  if (many && scans) {\n    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");\n',
                13)
    k = _insert(k, "  int32_t rank_sum = 0, batch_cnt = 0;\n", 12)
    for anchor in ("    scan_small(d, experts_per_rank, L, batch_cnt, rank_sum, true, cnt_ws,\n"
                   "               num_tokens_per_expert, num_tokens_per_rank, rank_tok_off, "
                   "expert_offsets,\n               rank_offsets);\n  } else if (!kColumns && many) {",
                   "      scan_small(d, experts_per_rank, L, batch_cnt, rank_sum, true, cnt_ws,\n"
                   "                 num_tokens_per_expert, num_tokens_per_rank, rank_tok_off, "
                   "expert_offsets,\n                 rank_offsets);\n    } else {"):
        k = _insert(k, anchor, 8, after=False)
    k = _insert(k, "  if (live) token_outputs<K>(d, t, L, ex, rmask, is_token_in_rank, slot_rank);\n"
                   "  if (by_column) {", 9, after=False)
    k = _insert(k, "  if (tid == 0) {\n    write_header(header, d, ntiles);", 10, after=False)
    k = k.rstrip()
    if not k.endswith("}"):
        raise SystemExit("layout_phases: unexpected end of layout_kernel")
    k = k[:-1] + "  FLUSH;\n}\n\n"
    src = src[:a] + k + src[b:]
    p = src.index("namespace ep {")
    return (src[:p] + "__device__ unsigned long long *g_ts;\n"
            "__shared__ unsigned long long s_ts[16];\n"
            "#define FLUSH if (threadIdx.x == 0 && g_ts != nullptr) "
            "for (int q_ = 0; q_ < 16; ++q_) g_ts[blockIdx.x * 16 + q_] = s_ts[q_]\n" + src[p:])


HARNESS = r'''
#include "ep_kernels.hip"
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
using namespace ep;
static const int kSlots[] = {@SLOTS@};
static const char *kNames[] = {@NAMES@};
static const int kScanner[] = {@SCANNER@};
static int run(int T, int k, int E, int R) {
  const Dims d{T, 128, k, E, R, 1};
  std::vector<int32_t> ids((size_t)T * k);
  std::mt19937 g(3);
  std::vector<int> pool(E);
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) pool[e] = e;
    for (int j = 0; j < k; ++j) {
      std::uniform_int_distribution<int> u(j, E - 1);
      std::swap(pool[j], pool[u(g)]);
      ids[(size_t)t * k + j] = pool[j];
    }
  }
  const WorkspaceLayout w = workspace_layout(T, k, E, R);
  const int grid = std::max(w.ntiles, 1);
  int32_t *idx, *ntpr, *ntpe, *eoff, *roff, *status; uint8_t *itir; char *ws;
  unsigned long long *ts;
  CK(hipMalloc(&idx, ids.size() * 4)); CK(hipMalloc(&ntpr, R * 4)); CK(hipMalloc(&ntpe, E * 4));
  CK(hipMalloc(&eoff, (E + 1) * 4)); CK(hipMalloc(&roff, (R + 1) * 4)); CK(hipMalloc(&status, 4));
  CK(hipMalloc(&itir, (size_t)T * R)); CK(hipMalloc(&ws, w.total));
  CK(hipMalloc(&ts, (size_t)grid * 16 * 8));
  CK(hipMemcpy(idx, ids.data(), ids.size() * 4, hipMemcpyHostToDevice));
  CK(hipMemset(status, 0, 4));
  CK(launch_workspace_init(ws, 0));
  CK(hipMemcpyToSymbol(HIP_SYMBOL(g_ts), &ts, sizeof(ts)));
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  const int nph = sizeof(kSlots) / sizeof(kSlots[0]);
  std::vector<unsigned long long> h((size_t)grid * 16);
  std::vector<double> evt;
  std::vector<std::vector<double>> ph(nph);
  for (int it = 0; it < 45; ++it) {
    CK(hipMemset(ts, 0, (size_t)grid * 128));
    CK(hipDeviceSynchronize());
    time_next_kernel(a, b);
    CK(launch_layout(d, idx, ntpr, ntpe, itir, eoff, roff, ws, status, 0, true));
    CK(hipEventSynchronize(b));
    float ms; CK(hipEventElapsedTime(&ms, a, b));
    CK(hipMemcpy(h.data(), ts, h.size() * 8, hipMemcpyDeviceToHost));
    if (it < 5) continue;
    evt.push_back(ms * 1e3);
    unsigned long long t0 = ~0ull; int scanner = -1;
    for (int i = 0; i < grid; ++i) { t0 = std::min(t0, h[i * 16]); if (h[i * 16 + 10]) scanner = i; }
    auto us = [&](unsigned long long v) { return v ? (double)(v - t0) / 100.0 : -1.0; };
    for (int p = 0; p < nph; ++p) {
      const int s = kSlots[p];
      if (kScanner[p]) { ph[p].push_back(scanner >= 0 ? us(h[scanner * 16 + s]) : -1); continue; }
      double m = -1;
      for (int i = 0; i < grid; ++i) if (h[i * 16 + s]) m = std::max(m, us(h[i * 16 + s]));
      ph[p].push_back(m);
    }
  }
  int st = -1; CK(hipMemcpy(&st, status, 4, hipMemcpyDeviceToHost));
  auto med = [](std::vector<double> v) { std::sort(v.begin(), v.end()); return v[v.size() / 2]; };
  printf("T=%d k=%d E=%d R=%d tiles=%d status=%d kernel events %.2f us\n", T, k, E, R, w.ntiles,
         st, med(evt));
  for (int p = 0; p < nph; ++p) {
    const double v = med(ph[p]);
    if (v >= 0) printf("  %-34s %6.2f us\n", kNames[p], v);
  }
  CK(hipFree(idx)); CK(hipFree(ntpr)); CK(hipFree(ntpe)); CK(hipFree(eoff)); CK(hipFree(roff));
  CK(hipFree(status)); CK(hipFree(itir)); CK(hipFree(ws)); CK(hipFree(ts));
  return st == 0 ? 0 : 1;
}
int main(int argc, char **argv) {
  for (int i = 1; i + 3 < argc; i += 4)
    if (run(atoi(argv[i]), atoi(argv[i + 1]), atoi(argv[i + 2]), atoi(argv[i + 3]))) return 1;
  return 0;
}
'''


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shapes", default="2048:8:256:8,4096:8:256:8,8192:6:64:8,16384:8:256:8",
                    help="comma-separated T:k:E:R batches (uniform distinct top-k routes)")
    ap.add_argument("--build-only", action="store_true", help="compile the probe, do not run it")
    args = ap.parse_args()
    shapes = [tuple(int(v) for v in s.split(":")) for s in args.shapes.split(",")]
    for T, k, E, R in shapes:
        if not (T > 0 and 1 <= k <= 32 and k <= E <= 1024 and E % R == 0 and R <= 64):
            raise SystemExit(f"layout_phases: unsupported shape {T}:{k}:{E}:{R}")
    with open(os.path.join(PKG, "csrc", "ep_kernels.hip")) as f:
        src = instrument(f.read())
    harness = (HARNESS.replace("@SLOTS@", ", ".join(str(s) for s, _, _ in PHASES))
               .replace("@NAMES@", ", ".join(f'"{n}"' for _, n, _ in PHASES))
               .replace("@SCANNER@", ", ".join("1" if w == "scanner" else "0" for _, _, w in PHASES)))
    with tempfile.TemporaryDirectory() as tmp:
        with open(os.path.join(tmp, "ep_kernels.hip"), "w") as f:
            f.write(src)
        with open(os.path.join(tmp, "main.hip"), "w") as f:
            f.write(harness)
        exe = os.path.join(tmp, "layout_phases")
        flags = [f for f in _build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
        cmd = [_build.hipcc(), *flags, "-I", tmp, "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(PKG, "csrc"), os.path.join(tmp, "main.hip"),
               os.path.join(PKG, "csrc", "ep_api.hip"), os.path.join(PKG, "csrc", "hbm_probe.hip"),
               "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise SystemExit("layout_phases: hipcc failed\n" + res.stdout + res.stderr)
        print(f"layout_phases: built the probe ({len(PHASES)} phases)", flush=True)
        if args.build_only:
            return
        argv = [str(v) for shape in shapes for v in shape]
        sys.exit(subprocess.run([exe, *argv]).returncode)


if __name__ == "__main__":
    main()
