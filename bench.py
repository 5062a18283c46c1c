"""Benchmark: one step = layout + dispatch + combine over one batch.

Workload (default): Prefill, 4096 tokens x 7168 hidden bf16, top-8 of 256
experts on 8 logical ranks, FP8 E4M3 dispatch with per-128 fp32 scales, bf16
combine of a synthetic expert output [T*k, 7168].  Inputs are resident in
HBM before timing starts.  The receive buffer is sized for the worst case
(T*k rows) and no count is read back, so a step makes no host round trip.

Throughput is algorithmic bytes per second (decimal GB), the bytes the
method must move:
  layout    T*k*4 (topk_idx) + T*R (rank mask) + 4*(E+R) (counts) + 4*(E+R+2) (offsets)
  dispatch  T*H*2 (x once) + T*k*8 (idx, gates) + M*row (row = 2H bf16, or
            H + 4H/128 FP8) + M*8 (row_src, recv gate) + T*k*4 (tok_slot_row)
  combine   M*2H (gathered rows) + T*k*8 (tok_slot_row, gates) + T*2H (out)
with M valid selections.  Workspace traffic is overhead and not counted.

`device_copy_gbps` (the runtime's copy of 1 GiB) and `hbm_probe_gbps` (a
streaming read / write / copy of 1 GiB with 16-byte accesses, streaming or
plain) give the rates this machine's HBM sustains, as context for the roofline.

`value` and `ms_per_step` are the median over K cold steps: before each,
an untimed read pass over 1 GiB evicts the 256 MB MALL and the L2s, so the
step reads its inputs from HBM with clean caches.  Each step is timed from
its first kernel's start to its last kernel's end by the kernels' own
events (ep_time_next_kernel), the span a kernel trace shows; the same
steps timed by events enqueued around them (which add the markers' own
overhead) are reported beside.  `kernel_us` and the roofline time each
call's kernels the same way over K more cold steps.  Also reported: warm steps
(back to back, part of x and the routes still in the MALL), and cold steps
after a write pass (`cold_dirty`, which also pays for writing back the
scratch's dirty lines).

Prints one JSON line.  --gpus above 1 exits: the library runs on one GPU per process.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "dispatch+combine HBM GB/s and % of peak; tokens/s at 4096x7168 top-8"
KERNEL_SOURCES = [os.path.join(ROOT, "combine_get_dispatch_amd", "csrc", f)
                  for f in ("ep_kernels.hip", "ep_internal.h")]


def algorithmic_bytes(w, M: int, fp8_input: bool = False, pad_rows: int = 0) -> dict:
    """fp8_input: rows arrive as E4M3 codes + scales (read once: H + H/32
    bytes per token instead of 2H).  pad_rows: alignment padding rows, which
    dispatch zero-fills (payload, scales, source and gate)."""
    T, H, k, E, R = w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks
    row = (H + 4 * (H // 128)) if w.fp8 else 2 * H
    layout = T * k * 4 + T * R + 4 * (E + R) + 4 * (E + R + 2)
    x_bytes = T * (H + 4 * (H // 128)) if fp8_input else T * H * 2
    dispatch = x_bytes + T * k * 8 + (M + pad_rows) * (row + 8) + T * k * 4
    combine = M * 2 * H + T * k * 8 + T * 2 * H
    return dict(layout=layout, dispatch=dispatch, combine=combine,
                total=layout + dispatch + combine)


def backward_bytes(w, M: int) -> dict:
    """Algorithmic bytes of the backward pair.
    dispatch_backward: M*2H (row gradients) + T*k*4 (tok_slot_row) + T*2H (grad_x)
    combine_backward:  T*2H (grad_out) + T*k*8 (tok_slot_row, gates) + M*2H (expert
                       outputs) + M*2H (row gradients) + T*k*4 (gate gradients)"""
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    db = M * 2 * H + T * k * 4 + T * 2 * H
    cb = T * 2 * H + T * k * 8 + 2 * M * 2 * H + T * k * 4
    return dict(dispatch_backward=db, combine_backward=cb, total=db + cb)


def ranked_bytes(w, M: int, Q: int) -> dict:
    """Algorithmic bytes of the non-expanded path with Q (token, rank) rows.
    dispatch_ranked: T*2H (x) + T*k*8 (idx, gates) + Q*row + Q*(4 + 8k)
                     (source, local slices) + T*R*4 + T*k*4 (both handles)
    expand:          Q*row + Q*8k (received rows and slices) + M*row + M*8
    combine_ranked:  M*2H + Q*8k + Q*4H (stage 1) + Q*4H + T*R*4 + T*2H (stage 2)"""
    T, H, k, R = w.num_tokens, w.hidden, w.num_topk, w.num_ranks
    row = (H + 4 * (H // 128)) if w.fp8 else 2 * H
    layout = T * k * 4 + T * R + 4 * (w.num_experts + R) + 4 * (w.num_experts + R + 2)
    disp = T * 2 * H + T * k * 8 + Q * row + Q * (4 + 8 * k) + T * R * 4 + T * k * 4
    exp = Q * row + Q * 8 * k + M * row + M * 8
    comb = M * 2 * H + Q * 8 * k + Q * 4 * H + Q * 4 * H + T * R * 4 + T * 2 * H
    return dict(layout=layout, dispatch_ranked=disp, expand=exp, combine_ranked=comb,
                total=layout + disp + exp + comb)


# The kernel and launcher each counter summary measures.
KERNEL_FUNCS = {"combine": ("combine_kernel", "launch_combine"),
                "dispatch": ("dispatch_kernel", "launch_dispatch"),
                "dispatch_bf16": ("dispatch_kernel", "launch_dispatch"),
                "layout": ("layout_kernel", "launch_layout")}


def split_functions(src: str) -> list:
    """Top-level pieces of a kernel source: each ends with a line that is a
    lone closing brace (a function) or brace-semicolon (a struct), and
    carries the comments above it."""
    pieces, cur = [], []
    for line in src.splitlines(keepends=True):
        cur.append(line)
        if line.rstrip() in ("}", "};"):
            pieces.append("".join(cur))
            cur = []
    if cur:
        pieces.append("".join(cur))
    return pieces


def _piece_name(piece: str):
    m = re.search(r"__global__\s+(?:__launch_bounds__\([^)]*\)\s+)?void\s+(\w+)\s*\(", piece)
    if m:
        return "kernel", m.group(1)
    m = re.search(r"\bhipError_t\s+(launch_\w+)\s*\(", piece)
    if m:
        return "launcher", m.group(1)
    return "helper", None


def _code_only(text: str) -> str:
    """The text without comments, trailing spaces or blank lines: edits to
    those do not change what is compiled."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


_IDENT = re.compile(r"\b[A-Za-z_]\w*\b")
_ATTRIBUTE = re.compile(r"\b(?:__\w+__|alignas)\s*\((?:[^()]|\([^()]*\))*\)")
_ONE_FUNCTION = re.compile(
    r"(?:template\s*<[^{};]*>\s*)?[^{};()]*?\b(\w+)\s*\([^{};]*\)\s*(?:const\s*)?\{\}")
_ONE_STRUCT = re.compile(r"(?:template\s*<[^{};]*>\s*)?struct\s+(\w+)[^{};]*\{\};")


def _outside_braces(code: str) -> str:
    """The code with the inside of every top-level brace pair dropped."""
    out, depth = [], 0
    for ch in code:
        if ch == "{":
            if depth == 0:
                out.append(ch)
            depth += 1
        elif ch == "}":
            depth -= 1
            if depth == 0:
                out.append(ch)
        elif depth == 0:
            out.append(ch)
    return "".join(out)


def _sole_definition(piece: str):
    """The name of the one function or struct a helper piece defines, or None
    when the piece holds anything besides (constants, typedefs, variables,
    preprocessor lines, a namespace, a second definition)."""
    top = _ATTRIBUTE.sub("", _outside_braces(_code_only(piece))).strip()
    for pattern in (_ONE_FUNCTION, _ONE_STRUCT):
        m = pattern.fullmatch(top)
        if m:
            return m.group(1)
    return None


def kernel_source_hash(kernel: str = None, src: str = None, extra: bytes = None) -> str:
    """Hash of what a kernel's measured behaviour depends on: the kernel's
    own function and launcher, the helper pieces of the kernel source
    (anything that is neither a kernel nor a launcher) that they use, the
    internal header and the compiler flags, all without comments.  A helper
    piece that defines one function or struct is used when its name appears
    in a piece already taken, followed to a fixed point; every other helper
    piece is always taken.  With kernel=None, the whole sources.  Editing
    another kernel, a helper only other kernels use, or a comment leaves a
    kernel's hash unchanged."""
    h = hashlib.sha256()
    if src is None:
        with open(KERNEL_SOURCES[0]) as f:
            src = f.read()
    if extra is None:
        extra = b""
        for path in KERNEL_SOURCES[1:]:
            with open(path) as f:
                extra += _code_only(f.read()).encode()
        from combine_get_dispatch_amd import _build

        extra += " ".join(_build.HIPCC_FLAGS).encode()
    h.update(extra)
    if kernel is None:
        h.update(_code_only(src).encode())
        return h.hexdigest()[:16]
    kname, lname = KERNEL_FUNCS[kernel]
    pieces = split_functions(src)
    taken = [False] * len(pieces)
    used = set()
    helpers = []
    for i, piece in enumerate(pieces):
        kind, name = _piece_name(piece)
        if name in (kname, lname):
            taken[i] = True
            used |= set(_IDENT.findall(_code_only(piece)))
        elif kind == "helper":
            helpers.append((i, _sole_definition(piece)))
    grew = True
    while grew:
        grew = False
        for i, name in helpers:
            if not taken[i] and (name is None or name in used):
                taken[i] = True
                used |= set(_IDENT.findall(_code_only(pieces[i])))
                grew = True
    for piece, take in zip(pieces, taken):
        if take:
            h.update(_code_only(piece).encode())
    return h.hexdigest()[:16]


def _read_kv(path: str) -> dict:
    out = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, _, val = line.partition("=")
                out[key.strip()] = val.strip()
    return out


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = _read_kv(path)
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


KERNEL_KEYS = {"layout": "layout_kernel", "dispatch": "dispatch_kernel<true>",
               "dispatch_bf16": "dispatch_kernel<false>", "combine": "combine_kernel"}


def phase_slices(warmup: int, steps: int) -> dict:
    """Which launches of each step kernel belong to which phase of the
    default command, in launch order: the warm-up steps, 3K cold steps
    (timed by kernel events, by markers, then per call), 3K warm steps
    (back to back, per step, per call) and min(K, 30) cold steps after a
    write pass."""
    W, K = warmup, steps
    return {"warmup": (0, W), "cold": (W, W + 3 * K), "warm": (W + 3 * K, W + 6 * K),
            "cold_dirty": (W + 6 * K, W + 6 * K + min(K, 30))}


def load_trace_cold_us(workload: str, kernel: str):
    """A kernel's average duration over the cold steps, from the committed
    kernel trace summary of the default command, if that summary was taken
    on the kernel's current sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.md")
    if not os.path.exists(path):
        return None
    rec = _read_kv(path)
    if rec.get(f"kernel_source_hash[{kernel}]") != kernel_source_hash(kernel):
        return None
    v = rec.get(f"cold_average_us[{kernel}]")
    return float(v) if v is not None else None


def _trace_rows(run_dir: str, name: str) -> list:
    import csv

    with open(os.path.join(run_dir, "trace", name)) as f:
        return list(csv.DictReader(f))


def _launch_table(run_dir: str, title: str, cmd: str) -> list:
    """Markdown lines: the command, then every kernel's statistics over all
    launches of a rocprofv3 --kernel-trace --stats run (run_dir/trace)."""
    lines = ["# Kernel durations, " + title, "", "Command:", "", "    " + cmd, "",
             "All launches:", "",
             "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in _trace_rows(run_dir, "ep_kernel_stats.csv"):
        lines.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    return lines


def mode_trace_summary(run_dir: str, mode: str, title: str, workload: str, cmd: str) -> None:
    """Summarise a kernel trace of one of the bench's other modes (`--ranked`,
    `--direction backward`) into profiles/<mode>_<workload>_kernel_trace.md:
    every kernel's statistics over all launches.  Those modes run their steps
    back to back (warm), so the averages hold no per-phase split."""
    lines = _launch_table(run_dir, f"{title}, {workload} workload", cmd)
    with open(os.path.join(ROOT, "profiles", f"{mode}_{workload}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"{mode} trace summary written for {workload}")


def trace_summary(run_dir: str, workload: str, cmd: str, warmup: int, steps: int) -> None:
    """Summarise a rocprofv3 --kernel-trace --stats run of the default
    command (run_dir/trace) into profiles/<workload>_kernel_trace.md: every
    kernel's statistics over all launches, and the step kernels' averages
    per phase (cold, warm, cold_dirty), taken from the launch order."""
    import statistics

    launches = sorted(_trace_rows(run_dir, "ep_kernel_trace.csv"),
                      key=lambda r: int(r["Dispatch_Id"]))
    lines = _launch_table(run_dir, workload + " workload", cmd)
    ph = phase_slices(warmup, steps)
    total = ph["cold_dirty"][1]
    lines += ["", f"Step kernels per phase, by launch order (warm-up {warmup} steps, then "
              f"cold {3 * steps}, warm {3 * steps}, cold after a write pass "
              f"{ph['cold_dirty'][1] - ph['cold_dirty'][0]}; average us):", "",
              "| kernel | cold | warm | cold_dirty |", "|---|---|---|---|"]
    kv = []
    for key, kname in KERNEL_KEYS.items():
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                for r in launches if kname in r["Kernel_Name"]]
        if not durs:
            continue
        if len(durs) != total:
            lines.append(f"| {key} | ({len(durs)} launches, expected {total}) | | |")
            continue
        avg = {p: statistics.mean(durs[a:b]) for p, (a, b) in ph.items() if b > a}
        lines.append(f"| {key} | {avg['cold']:.2f} | {avg['warm']:.2f} | "
                     f"{avg['cold_dirty']:.2f} |")
        kv += [f"cold_average_us[{key}] = {avg['cold']:.2f}",
               f"warm_average_us[{key}] = {avg['warm']:.2f}",
               f"kernel_source_hash[{key}] = {kernel_source_hash(key)}"]
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines + [""] + kv) + "\n")
    print(f"trace summary written for {workload}")


def pmc_summary(run_dir: str, workload: str, copy_mib: int, cmds: dict):
    """Summarise rocprofv3 counter runs under run_dir (fetch/, write/, plus
    trace/ for the durations) into profiles/: HBM bytes per launch from
    FETCH_SIZE / WRITE_SIZE scaled by what the counters read for a plain
    device copy of copy_mib MiB."""
    import csv
    import statistics

    def rows(sub, name):
        with open(os.path.join(run_dir, sub, name)) as f:
            return list(csv.DictReader(f))

    def per_kernel(sub):
        vals = {}
        for r in rows(sub, "ep_counter_collection.csv"):
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel("fetch"), per_kernel("write")
    copy_kib = copy_mib * 1024.0

    def copy_factor(vals):
        cands = [max(v) for k, v in vals.items() if "copyBuffer" in k]
        f = copy_kib / max(cands)
        # the counters read whole or half the copied bytes on this chip; any
        # other factor means the run held a copy of another size
        if not (0.9 <= f <= 2.2):
            raise SystemExit(f"copy counter factor {f:.4f} is implausible; was the only "
                             f"device copy the {copy_mib} MiB probe?")
        return f

    ff, wf = copy_factor(fetch), copy_factor(write)
    stats = {r["Name"]: r for r in rows("trace", "ep_kernel_stats.csv")}
    for key, kname in KERNEL_KEYS.items():
        fk = [k for k in fetch if kname in k]
        wk = [k for k in write if kname in k]
        if not fk or not wk:
            continue
        fkib = statistics.median(fetch[fk[0]])
        wkib = statistics.median(write[wk[0]])
        avg_ns = [float(r["AverageNs"]) for n, r in stats.items() if kname in n]
        body = [
            f"# HBM traffic of {kname}, {workload} workload (rocprofv3 counters)",
            "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch (median over dispatches),",
            f"# scaled by copy_mib*1024 / (counter of a plain {copy_mib} MiB device copy).",
            f"# trace command: {cmds['trace']}",
            f"# fetch command: {cmds['fetch']}",
            f"# write command: {cmds['write']}",
            f"kernel = {fk[0].split('(')[0]}",
            f"fetch_size_kib = {fkib:.1f}",
            f"write_size_kib = {wkib:.1f}",
            f"copy_fetch_factor = {ff:.4f}",
            f"copy_write_factor = {wf:.4f}",
            f"hbm_read_bytes_per_launch = {fkib * ff * 1024:.0f}",
            f"hbm_write_bytes_per_launch = {wkib * wf * 1024:.0f}",
            f"hbm_bytes_per_launch = {(fkib * ff + wkib * wf) * 1024:.0f}",
            f"average_duration_us = {avg_ns[0] / 1e3:.2f}" if avg_ns else "average_duration_us = nan",
            f"kernel_source_hash = {kernel_source_hash(key)}",
        ]
        with open(os.path.join(ROOT, "profiles", f"{key}_{workload}_hbm_traffic.txt"), "w") as f:
            f.write("\n".join(body) + "\n")
    print(f"counter summaries written for {workload} (copy factors fetch {ff:.4f}, "
          f"write {wf:.4f})")


def short_kernel_name(name: str) -> str:
    """A profiler's demangled kernel name without its return type and
    argument list; an anonymous namespace keeps a readable tag."""
    name = name.replace("(anonymous namespace)::", "anon::")
    return name.split("(")[0].replace("void ", "")


def logical_network_bytes(w, b) -> dict:
    """What an expert-parallel group of R GPUs would send over its links for
    this batch, as DeepEP counts it: one row per (token, destination rank)
    in dispatch (the payload row: bf16, or E4M3 codes + per-128 scales) and
    one bf16 row back per (token, rank) in combine.  Nothing here moves
    these bytes; they are reported beside the HBM bytes.  `remote` leaves
    out each token's own rank, with token t owned by rank t*R/T."""
    import numpy as np

    T, H, R = w.num_tokens, w.hidden, w.num_ranks
    mask = b.is_token_in_rank.cpu().numpy().astype(bool)
    rows = int(mask.sum())
    own = np.arange(T, dtype=np.int64) * R // max(T, 1)
    remote = rows - int(mask[np.arange(T), own].sum()) if T else 0
    row_b = H + 4 * (H // 128) if w.fp8 else 2 * H
    return {"rows": rows, "rows_per_token": round(rows / max(T, 1), 4),
            "expanded_rows_per_token": round(int(b.num_tokens_per_expert.sum().item())
                                             / max(T, 1), 4),
            "dispatch_bytes": rows * row_b, "combine_bytes": rows * 2 * H,
            "remote_rows": remote, "remote_dispatch_bytes": remote * row_b,
            "remote_combine_bytes": remote * 2 * H}


def run_receipt(w, inp, b, dev) -> dict:
    """What identifies the run: toolchain and GPU, the workload's seed, and
    the route's shape (expert load skew; the share of selections whose
    expert lives on the token's own logical rank, with token t owned by
    rank t*R/T)."""
    import subprocess

    import numpy as np
    import torch

    props = torch.cuda.get_device_properties(dev)
    try:
        sha = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, text=True,
                             capture_output=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        sha = None
    idx = inp["topk_idx"]
    T, E, R = w.num_tokens, w.num_experts, w.num_ranks
    valid = idx >= 0
    own = (np.arange(T, dtype=np.int64) * R // T)[:, None]
    local = (idx // (E // R) == own) & valid
    load = b.num_tokens_per_expert.cpu().numpy()
    return {"git": sha, "torch": torch.__version__, "hip": torch.version.hip,
            "gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "host_cpu": host_cpu_model(), "host_cpus": host_cpus(),
            "seed": w.seed, "max_over_mean_expert_load": round(float(load.max() / load.mean()), 3),
            "local_rank_fraction": round(float(local.sum() / max(1, valid.sum())), 4)}


def step_outputs(b) -> dict:
    """Host copies of what the last timed step left in the buffers."""
    import numpy as np
    import torch

    rows = int(b.expert_offsets[-1].item())
    got = {n: getattr(b, n).cpu().numpy() for n in
           ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
            "expert_offsets", "rank_offsets", "tok_slot_row")}
    got["row_src"] = b.row_src[:rows].cpu().numpy()
    got["recv_weights"] = b.recv_weights[:rows].cpu().numpy()
    rx = b.recv_x[:rows].cpu()
    got["recv_x"] = rx.numpy() if b.fp8 else rx.view(torch.int16).numpy().view(np.uint16)
    got["recv_scales"] = b.recv_scales[:rows].cpu().numpy() if b.fp8 else None
    got["out"] = b.out.cpu().view(torch.int16).numpy().view(np.uint16)
    return got


def compare_step(got: dict, lay: dict, d: dict, ref_out) -> dict:
    """The timed step's outputs against the oracle's for the same batch:
    layout, handle, rows and scales bit for bit, combine as bf16 bits."""
    import numpy as np

    rows = int(lay["expert_offsets"][-1])
    same = lambda a, b: bool(a is None and b is None or np.array_equal(a, b))
    ok = {
        "layout": all(same(got[n], lay[n]) for n in
                      ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
                       "expert_offsets", "rank_offsets")),
        "handle": same(got["tok_slot_row"], d["tok_slot_row"])
                  and same(got["row_src"], d["row_src"][:rows])
                  and same(got["recv_weights"].view(np.uint32),
                           d["recv_weights"][:rows].view(np.uint32)),
        "rows": same(got["recv_x"], d["recv_x"][:rows])
                and (d["recv_scales"] is None
                     or same(got["recv_scales"].view(np.uint32),
                             d["recv_scales"][:rows].view(np.uint32))),
        "combine_bits": same(got["out"], ref_out),
    }
    ok["all"] = all(ok.values())
    return ok


def cpu_baseline(w, inp, budget_s: float, got: dict | None = None):
    """The CPU oracle as it stands (single-threaded C), timed on this host on
    whole steps of the same batch, repeated until about budget_s seconds.
    With got (the timed GPU step's outputs), the last oracle step's results
    are also compared with them."""
    import oracle

    reps, t0 = 0, time.perf_counter()
    while True:
        lay = oracle.layout(inp["topk_idx"], w.num_experts, w.num_ranks, w.alignment)
        d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_weights"], w.num_experts,
                            w.num_ranks, w.alignment, fp8=w.fp8)
        ref_out, _ = oracle.combine(inp["y"], d["tok_slot_row"], inp["topk_weights"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 8:
            break
    M = int(lay["expert_offsets"][-1])
    b = algorithmic_bytes(w, M)["total"]
    rec = dict(value=round(b * reps / el / 1e9, 3), unit="GB/s", cores=1, kind="oracle",
               sample=f"{reps} full {w.name} step(s) (layout+dispatch+combine, "
                      f"{w.num_tokens} tokens) in {el:.1f} s, single-threaded C",
               tokens_per_s=round(w.num_tokens * reps / el, 1))
    if got is not None:
        rec["timed_step_matches_oracle"] = compare_step(got, lay, d, ref_out)
    return rec


def host_cpus() -> int:
    """Cores this process may run on (its affinity mask), capped at 16, the
    host share that one GPU's jobs get."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def host_cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_all_cores(w, inp, budget_s: float, threads: int):
    """The same oracle, unchanged, on every available core: `threads` host
    threads each run whole steps (layout, dispatch, combine) of the batch
    until about budget_s seconds have passed.  ctypes releases the GIL
    around the C calls, so the steps run in parallel; each thread keeps its
    own outputs.  The rate is the aggregate over all threads."""
    import threading

    import oracle

    oracle.layout(inp["topk_idx"][:1], w.num_experts, w.num_ranks, w.alignment)  # load once
    done = [0] * threads
    t0 = time.perf_counter()

    def work(i):
        while True:
            oracle.layout(inp["topk_idx"], w.num_experts, w.num_ranks, w.alignment)
            d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_weights"], w.num_experts,
                                w.num_ranks, w.alignment, fp8=w.fp8)
            oracle.combine(inp["y"], d["tok_slot_row"], inp["topk_weights"])
            del d
            done[i] += 1
            if time.perf_counter() - t0 >= budget_s:
                return

    pool = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    el = time.perf_counter() - t0
    reps = sum(done)
    lay = oracle.layout(inp["topk_idx"], w.num_experts, w.num_ranks, w.alignment)
    b = algorithmic_bytes(w, int(lay["expert_offsets"][-1]))["total"]
    return dict(value=round(b * reps / el / 1e9, 3), unit="GB/s", cores=threads,
                kind="oracle", sample=f"{reps} full {w.name} step(s) on {threads} threads at "
                                      f"once (one step per thread at a time) in {el:.1f} s",
                tokens_per_s=round(w.num_tokens * reps / el, 1))


def run_backward(args, w, b, x, idx, wts, y, inp, dev, stream):
    """Time the backward pair over one batch: gradient w.r.t. the receive
    rows -> grad_x (dispatch backward), and grad_out -> row and gate
    gradients (combine backward), after one forward layout + dispatch."""
    import numpy as np
    import torch

    import ep_workloads as W

    g = W.normal_bf16(np.random.default_rng(100 + w.seed), (w.num_tokens, w.hidden))
    g_d = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(dev)
    b.layout(idx)
    b.dispatch(x, idx, wts)
    b.check_status()
    M = int(b.expert_offsets[-1].item())
    grad_x = torch.empty_like(b.out)
    gy = torch.empty((b.capacity, w.hidden), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((w.num_tokens, w.num_topk), dtype=torch.float32, device=dev)

    def step():
        b.dispatch_backward(y, grad_x)
        b.combine_backward(g_d, wts, y, gy, gw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    names = ("dispatch_backward", "combine_backward")
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in names}
    for i in range(args.steps):
        for n, fn in zip(names, (lambda: b.dispatch_backward(y, grad_x),
                                 lambda: b.combine_backward(g_d, wts, y, gy, gw))):
            ev[n][i][0].record(stream)
            fn()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    per_us = {n: float(np.mean([a.elapsed_time(c) for a, c in ev[n]])) * 1e3 for n in names}
    by = backward_bytes(w, M)
    gbps = by["total"] / (ms / 1e3) / 1e9
    rec = {
        "metric": "backward (dispatch_backward + combine_backward) HBM GB/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "tokens_per_s": round(w.num_tokens / (ms / 1e3), 1),
        "config": {"workload": w.name, "tokens": w.num_tokens, "hidden": w.hidden,
                   "topk": w.num_topk, "experts": w.num_experts, "valid_selections": M},
        "algorithmic_bytes_per_step": by,
        "kernel_us": {n: round(v, 2) for n, v in per_us.items()},
        "kernel_roofline_frac": {n: round(by[n] / (per_us[n] / 1e6) / 1e9 / PEAK_HBM_GBPS, 4)
                                 for n in names},
    }
    print(json.dumps(rec), flush=True)


def run_ranked(args, w, b, x, idx, wts, y, stream):
    """Time the non-expanded path over one batch: layout, one row per
    (token, rank), receiver-side expand to the expert-major layout, and the
    combine through fp32 per-rank partials."""
    import numpy as np
    import torch

    names = ("layout", "dispatch_ranked", "expand", "combine_ranked")
    calls = (lambda: b.layout(idx), lambda: b.dispatch_ranked(x, idx, wts), lambda: b.expand(),
             lambda: b.combine_ranked(y))
    for _ in range(args.warmup):
        for fn in calls:
            fn()
    b.check_status()
    M = int(b.expert_offsets[-1].item())
    Q = int(b.rank_token_offsets[-1].item())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        for fn in calls:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in names}
    for i in range(args.steps):
        for n, fn in zip(names, calls):
            ev[n][i][0].record(stream)
            fn()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    b.check_status()
    per_us = {n: float(np.mean([a.elapsed_time(c) for a, c in ev[n]])) * 1e3 for n in names}
    by = ranked_bytes(w, M, Q)
    gbps = by["total"] / (ms / 1e3) / 1e9
    rec = {
        "metric": "non-expanded dispatch + expand + ranked combine HBM GB/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "tokens_per_s": round(w.num_tokens / (ms / 1e3), 1),
        "config": {"workload": w.name, "tokens": w.num_tokens, "hidden": w.hidden,
                   "topk": w.num_topk, "experts": w.num_experts, "logical_ranks": w.num_ranks,
                   "valid_selections": M, "token_rank_rows": Q,
                   "rows_per_token": round(Q / max(w.num_tokens, 1), 4)},
        "algorithmic_bytes_per_step": by,
        "kernel_us": {n: round(v, 2) for n, v in per_us.items()},
        "kernel_roofline_frac": {n: round(by[n] / (per_us[n] / 1e6) / 1e9 / PEAK_HBM_GBPS, 4)
                                 for n in names},
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter scale)")
    ap.add_argument("--fp8-input", action="store_true",
                    help="dispatch pre-quantised rows (E4M3 codes + scales) instead of bf16")
    ap.add_argument("--ranked", action="store_true",
                    help="time the non-expanded path (dispatch_ranked + expand + "
                         "combine_ranked; its own JSON line)")
    ap.add_argument("--alignment", type=int, default=0,
                    help="expert alignment A (padded, zero-filled segments) instead of the "
                         "workload's")
    ap.add_argument("--replay", action="store_true",
                    help="cached route: one layout, then steps of dispatch + combine")
    ap.add_argument("--fused", action="store_true",
                    help="layout and dispatch in one call (ep_layout_dispatch: one launch up to "
                         "256 tokens)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one forward step as a HIP graph and time its replays")
    ap.add_argument("--direction", choices=("forward", "backward"), default="forward",
                    help="backward times ep_dispatch_backward + ep_combine_backward (its own "
                         "JSON line, not the forward metric)")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None,
                    help="summarise rocprofv3 trace/fetch/write runs in DIR into profiles/")
    ap.add_argument("--trace-summary", metavar="DIR", default=None,
                    help="summarise the rocprofv3 kernel trace run in DIR/trace into profiles/ "
                         "(--warmup and --steps as in the traced command)")
    args = ap.parse_args()

    if args.trace_summary and (args.ranked or args.direction == "backward"):
        mode, title, flag = (("ranked", "non-expanded path", "--ranked") if args.ranked else
                             ("backward", "backward pair", "--direction backward"))
        mode_trace_summary(
            args.trace_summary, mode, title, args.workload,
            "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o ep -- "
            f"python3 bench.py {flag} --no-cpu-baseline"
            + ("" if args.workload == "prefill" else f" --workload {args.workload}"))
        return
    if args.pmc_summary or args.trace_summary:
        base = (f"python3 bench.py --workload {args.workload} --steps 3 --warmup 1 "
                f"--no-cpu-baseline --copy-probe-mib 256")
        cmds = {
            "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o ep -- "
                     + ("python3 bench.py" if args.workload == "prefill"
                        else f"python3 bench.py --workload {args.workload}"),
            "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o ep -- {base}",
            "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o ep -- {base}",
        }
        run_dir = args.pmc_summary or args.trace_summary
        trace_summary(run_dir, args.workload, cmds["trace"], args.warmup, args.steps)
        if args.pmc_summary:
            pmc_summary(run_dir, args.workload, 256, cmds)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the library runs on one GPU per process; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import combine_get_dispatch_amd as ep
    import ep_workloads as W

    w = W.WORKLOADS[args.workload]
    if args.alignment:
        import dataclasses

        w = dataclasses.replace(w, alignment=args.alignment)
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = W.generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    wts = torch.from_numpy(inp["topk_weights"]).to(dev)
    y = torch.from_numpy(inp["y"].view(np.int16)).view(torch.bfloat16).to(dev)
    b = ep.EpBuffers(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                     w.alignment, fp8=w.fp8, device=dev)
    stream = torch.cuda.current_stream()
    if args.fp8_input and not w.fp8:
        raise SystemExit("--fp8-input needs an FP8 workload (prefill or large)")
    if args.fp8_input:
        rng = np.random.default_rng(500 + w.seed)
        codes = torch.from_numpy(rng.integers(0, 256, (w.num_tokens, w.hidden),
                                              dtype=np.uint8)).to(dev)
        scales = torch.from_numpy(rng.random((w.num_tokens, w.hidden // 128))
                                  .astype(np.float32)).to(dev)

    def do_dispatch():
        if args.fp8_input:
            b.dispatch_fp8_input(codes, scales, idx, wts)
        else:
            b.dispatch(x, idx, wts)

    if args.fused and args.fp8_input:
        raise SystemExit("--fused takes bf16 or quantising dispatch, not pre-quantised rows")

    def step():
        if args.fused:
            b.layout_dispatch(x, idx, wts)
        elif args.replay:
            do_dispatch()  # cached route: the layout ran once, before warm-up
        else:
            b.layout(idx)
            do_dispatch()
        b.combine(y, wts)

    if args.replay:
        b.layout(idx)

    if args.direction == "backward":
        run_backward(args, w, b, x, idx, wts, y, inp, dev, stream)
        return
    if args.ranked:
        run_ranked(args, w, b, x, idx, wts, y, stream)
        return

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    b.check_status()
    M = int(b.num_tokens_per_expert.sum().item())
    pad_rows = int(b.expert_offsets[-1].item()) - M

    eager_step = step
    if args.graph:
        # one step captured as a HIP graph; replays launch its kernels without
        # the host's per-call launch overhead
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            eager_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        b.check_status()

    # per call (the kernel each call launches)
    if args.fused:
        names = ("layout_dispatch", "combine")
        fns = (lambda: b.layout_dispatch(x, idx, wts), lambda: b.combine(y, wts))
    elif args.replay:
        names = ("dispatch", "combine")
        fns = (do_dispatch, lambda: b.combine(y, wts))
    else:
        names = ("layout", "dispatch", "combine")
        fns = (lambda: b.layout(idx), do_dispatch, lambda: b.combine(y, wts))

    # Cold steps: an untimed pass over 1 GiB before each step evicts the
    # 256 MB MALL and the L2s, so the step reads its inputs from HBM.  A read
    # pass ("cold") leaves the caches clean; a write pass ("cold_dirty")
    # leaves them dirty, so the step also pays for writing back the scratch's
    # lines.  Warm steps run back to back and find part of the previous
    # step's x and routes in the MALL.
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)

    def evict(kind, i):
        if kind == "read":
            scratch.amax()
        elif kind == "write":
            scratch.fill_(i)

    def new_pairs(n, create):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n)]
        if create:  # the events must exist on the device before a kernel records them
            for a, c in pairs:
                a.record(stream)
                c.record(stream)
            torch.cuda.synchronize()
        return pairs

    def timed_steps(n, kind, markers=False):
        """Per-step microseconds of n steps.  By default a step is timed from
        the start of its first kernel to the end of its last, by the
        kernels' own events (ep_time_next_kernel); with markers (and for
        graph replays), by events enqueued before and after the step, which
        add the markers' own overhead."""
        markers = markers or args.graph
        pairs = new_pairs(n, not markers)
        for i, (a, c) in enumerate(pairs):
            evict(kind, i)
            if markers:
                a.record(stream)
                step()
                c.record(stream)
            else:
                for j, fn in enumerate(fns):
                    if j == 0:
                        ep.ep_time_next_kernel(a, c if len(fns) == 1 else None)
                    elif j == len(fns) - 1:
                        ep.ep_time_next_kernel(None, c)
                    fn()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(c) * 1e3 for a, c in pairs])

    def timed_kernels(n, kind):
        """Mean duration (us) of each call's kernel over n steps, timed by
        the kernel's own start and stop events (ep_time_next_kernel)."""
        ev = {nm: new_pairs(n, True) for nm in names}
        for i in range(n):
            evict(kind, i)
            for nm, fn in zip(names, fns):
                ep.ep_time_next_kernel(*ev[nm][i])
                fn()
        torch.cuda.synchronize()
        return {nm: float(np.mean([a.elapsed_time(c) for a, c in ev[nm]])) * 1e3
                for nm in names}

    def dist(us):
        return {"median": round(float(np.median(us)), 2), "mean": round(float(np.mean(us)), 2),
                "p10": round(float(np.percentile(us, 10)), 2),
                "p90": round(float(np.percentile(us, 90)), 2), "n": int(len(us))}

    # The headline: K cold steps (read eviction).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold_us = timed_steps(args.steps, "read")
    wall = time.perf_counter() - t0
    ms_per_step = float(np.median(cold_us)) / 1e3
    print(f"bench: {args.steps} cold steps, median {ms_per_step * 1e3:.1f} us/step",
          file=sys.stderr, flush=True)
    cold_marker_us = timed_steps(args.steps, "read", markers=True)
    per_us = timed_kernels(args.steps, "read")
    b.check_status()

    # Warm: K steps back to back (one event pair), then per step and per call.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    warm_mean_us = e0.elapsed_time(e1) / args.steps * 1e3
    warm_us = timed_steps(args.steps, None)
    per_us_warm = timed_kernels(args.steps, None)
    dirty_us = timed_steps(min(args.steps, 30), "write")
    b.check_status()
    del scratch
    step_us = {"cold": dist(cold_us), "cold_marker_events": dist(cold_marker_us),
               "warm": dict(dist(warm_us), back_to_back_mean=round(warm_mean_us, 2)),
               "cold_dirty": dist(dirty_us)}

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Context: the runtime's own device-to-device copy of 1 GiB on this machine
    # (read + write bytes per second).  Counter runs (--copy-probe-mib) skip
    # it: their only copy must be the one of known size.
    copy_gbps = None
    if not args.copy_probe_mib:
        csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        cdst.copy_(csrc)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            cdst.copy_(csrc)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = round(2 * (1 << 30) * 5 / (c0.elapsed_time(c1) / 1e3) / 1e9, 1)
        del csrc, cdst

    # Context: the box's streaming read / write / copy rates over 1 GiB with
    # the kernels' own 16-byte accesses, streaming (nt) or plain.
    hbm_probe = None
    if not args.copy_probe_mib:
        nb = 1 << 30
        pa = torch.ones(nb, dtype=torch.uint8, device=dev)
        pb = torch.empty_like(pa)
        hbm_probe = {}
        for name, kind, nt, moved in (("read_nt", ep.EP_PROBE_READ, 1, nb),
                                      ("read", ep.EP_PROBE_READ, 0, nb),
                                      ("write_nt", ep.EP_PROBE_WRITE, 1, nb),
                                      ("write", ep.EP_PROBE_WRITE, 0, nb),
                                      ("copy_nt", ep.EP_PROBE_COPY, 1, 2 * nb),
                                      ("copy", ep.EP_PROBE_COPY, 0, 2 * nb)):
            best = 0.0
            for wgs in (1024, 4096, 16384, 65536):
                ep.ep_hbm_probe(kind, nt, wgs, pa, pb, nb)
                p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                p0.record(stream)
                for _ in range(5):
                    ep.ep_hbm_probe(kind, nt, wgs, pa, pb, nb)
                p1.record(stream)
                torch.cuda.synchronize()
                best = max(best, moved * 5 / (p0.elapsed_time(p1) / 1e3) / 1e9)
            hbm_probe[name] = round(best, 1)
        del pa, pb

    receipt = run_receipt(w, inp, b, dev)
    net_bytes = logical_network_bytes(w, b)
    by = algorithmic_bytes(w, M, args.fp8_input, pad_rows)
    if args.fused:
        by["layout_dispatch"] = by["layout"] + by["dispatch"]
    if args.replay:
        by["total"] -= by["layout"]
    step_s = ms_per_step / 1e3
    gbps = by["total"] / step_s / 1e9
    dom = max(names[-2:], key=lambda n: per_us[n])
    achieved = by[dom] / (per_us[dom] / 1e6) / 1e9
    # the committed counter and trace summaries are of the default command only
    default_mode = not (args.fp8_input or args.alignment or args.replay or args.fused
                        or args.graph)
    traffic_key = "dispatch_bf16" if dom == "dispatch" and not w.fp8 else dom
    traffic = load_traffic(w.name, traffic_key) if default_mode else None
    trace_us = load_trace_cold_us(w.name, traffic_key) if default_mode else None
    rec = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3 dispatch (fp32 quantiser), bf16 combine with fp32 accumulation"
                  if w.fp8 and not args.fp8_input else
                  "e4m3 codes copied, bf16 combine with fp32 accumulation" if args.fp8_input
                  else "bf16 dispatch (bit copy), bf16 combine with fp32 accumulation"),
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.num_tokens} tokens x {w.hidden} hidden, "
                               f"top-{w.num_topk} of {w.num_experts} experts on "
                               f"{w.num_ranks} logical ranks, "
                               f"{'FP8 E4M3' if w.fp8 else 'bf16'} dispatch, bf16 combine",
                   "tokens": w.num_tokens, "hidden": w.hidden, "topk": w.num_topk,
                   "experts": w.num_experts, "logical_ranks": w.num_ranks,
                   "dispatch_payload": ("fp8_e4m3 (pre-quantised input)" if args.fp8_input
                                        else "fp8_e4m3" if w.fp8 else "bf16"),
                   "valid_selections": M,
                   "launch": "hip_graph" if args.graph else "eager",
                   "layout": ("fused with dispatch (one launch)" if args.fused
                              else "once, route cached" if args.replay else "own launch"),
                   "alignment": w.alignment, "padding_rows": pad_rows},
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "tokens_per_s": round(w.num_tokens / step_s, 1),
        "algorithmic_bytes_per_step": by,
        "timing": ("value and ms_per_step: median of K cold steps (an untimed read pass "
                   "over 1 GiB evicts the MALL and L2s before each), each timed from its first "
                   "kernel's start to its last kernel's end by the kernels' own events; "
                   "step_us.cold_marker_events times K more with events enqueued around the "
                   "step (their overhead included); kernel_us: each call timed the same way "
                   "over K more cold steps"),
        "kernel_us": {n: round(v, 2) for n, v in per_us.items()},
        "kernel_us_warm": {n: round(v, 2) for n, v in per_us_warm.items()},
        "kernel_roofline_frac": {n: round(by[n] / (per_us[n] / 1e6) / 1e9 / PEAK_HBM_GBPS, 4)
                                 for n in names},
        "step_us": step_us,
        "warm_value": round(by["total"] / (warm_mean_us / 1e6) / 1e9, 1),
        "cold_dirty_value": round(by["total"] / (step_us["cold_dirty"]["median"] / 1e6) / 1e9,
                                  1),
        "receipt": receipt,
        "logical_network_bytes": net_bytes,
        "device_copy_gbps": copy_gbps,
        "hbm_probe_gbps": hbm_probe,
        "host_wall_s": round(wall, 4),
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel_us": round(per_us[dom], 2),
            "timing": "kernel start/stop events, cold steps",
            "trace_us": trace_us,
            "trace_frac": (round(by[dom] / (trace_us / 1e6) / 1e9 / PEAK_HBM_GBPS, 4)
                           if trace_us else None),
            "trace_file": f"profiles/{w.name}_kernel_trace.md" if trace_us else None,
        },
    }
    if not args.no_cpu_baseline and not args.fp8_input:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        got = step_outputs(b)
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, got)
        del got
        if not rec["cpu_baseline"]["timed_step_matches_oracle"]["all"]:
            print("bench: WARNING: the timed step's outputs differ from the oracle's",
                  file=sys.stderr, flush=True)
        n = host_cpus()
        if n > 1:
            print(f"bench: CPU oracle baseline on {n} threads", file=sys.stderr, flush=True)
            rec["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(w, inp, args.cpu_budget,
                                                                      n)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
