"""Benchmark of the target-verify path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload high_batch]

A step is one pass of the whole path for one batch: tv_build_tree_mask,
tv_verify_attn (prefix stream, merge with tail and chain, scratch pad),
tv_accept and tv_refresh_state.  Inputs are seeded synthetic data resident in HBM
before timing; the persistent state evolves from step to step as it would while
decoding.  Prints one JSON line:

  value          verified tree tokens per second (B*D per step / step time)
  roofline       the attention kernel (prefix stream + tail + chain): algorithmic
                 bytes per launch (every committed pool entry's K and V once, the
                 tail, Q, O, tree K/V, plan) over its average launch time from HIP
                 events on its stream, vs 8 TB/s
  cpu_baseline   the fp64 oracle timed on this host for a bounded sample of the
                 same workload (rank 0, N = 1 only)
  read_ceiling   a plain HIP read-reduce over 4 GiB on the same device (the practical
                 HBM read ceiling) and the attention kernel's fraction of it

    python bench.py --sweep OUT.md [--steps K] [--warmup W]

runs the long-context budget sweep instead (see sweep()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak (AMD's published figure)
N_INPUT_SETS = 4        # distinct per-step input sets, rotated


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first (kernel times drift for the first ~10 ms of a busy period)")
    ap.add_argument("--workload", default="high_batch")
    ap.add_argument("--parts", type=int, default=0, help="prefix-stream workgroups (0 = library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-in-place", action="store_true",
                    help="scratch pad without the in-place chain: the refresh copies every committed entry")
    ap.add_argument("--defer-coarse", action="store_true",
                    help="the coarsest level gets no scratch states; the refresh updates it from the accepted path")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the draft-tree, draft-attention and paged-pool measurements (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="time budget of the oracle sample")
    ap.add_argument("--summarize-profiles", default="", metavar="DIR",
                    help="write profiles/*.md and the traffic JSON from rocprofv3 csv runs in DIR "
                         "(kt/, FETCH_SIZE/, WRITE_SIZE/, copy_FETCH_SIZE/, copy_WRITE_SIZE/, kt.txt)")
    ap.add_argument("--sweep", default="", metavar="OUT_MD",
                    help="run the long-context budget sweep instead (D 5..8 x batch 1..64 x top-k 1, 2 at a "
                         "131072-token prefix) and write its table to OUT_MD; one JSON line per point")
    ap.add_argument("--sweep-batches", default="1,4,16,64", help="batch sizes of the sweep (comma-separated)")
    ap.add_argument("--summarize-sweep-traces", default="", metavar="DIR",
                    help="write profiles/step_long_context_kernel_trace.md from rocprofv3 kernel-trace csv "
                         "runs of the sweep, one per batch size, in DIR/b<B>/")
    ap.add_argument("--summarize-step-trace", default="", metavar="DIR",
                    help="write profiles/step_<workload>_kernel_trace.md from a rocprofv3 kernel-trace csv run "
                         "of the STEP_TRACE_CMD command in DIR/")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (to scale HBM byte counters)")
    return ap.parse_args()


class TimingEvent:
    """A HIP event for timing only (hipEventDisableSystemFence): recording it skips the
    system-scope cache writeback and invalidation a default event performs, which would
    otherwise add several microseconds around the kernel it brackets."""
    _hip = None

    def __init__(self):
        import ctypes
        import tree_speculative_decoding_amd as tv
        if TimingEvent._hip is None:  # the HIP runtime libtv.so runs on (symbols via its handle)
            TimingEvent._hip = tv.lib()
        self._ct = ctypes
        h = ctypes.c_void_p()
        if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(0x20000000)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.handle = h.value

    def elapsed_ms(self, stop: "TimingEvent") -> float:
        ms = self._ct.c_float()
        if TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self._ct.c_void_p(self.handle),
                                                self._ct.c_void_p(stop.handle)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        # (at interpreter exit the module's globals may already be gone: reach the runtime
        # through the instance's class and give up quietly)
        hip = getattr(type(self), "_hip", None)
        handle = getattr(self, "handle", None)
        if hip is not None and handle:
            try:
                hip.hipEventDestroy(self._ct.c_void_p(handle))
            except Exception:
                pass


def calibrate_copy(mib: int):
    """Plain copies of a known size: what FETCH_SIZE / WRITE_SIZE read for them gives the
    counters' scale (bytes counted per byte moved)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 5}), flush=True)


PROFILE_BENCH = "python3 bench.py --gpus 1 --steps 20 --warmup 5"  # the headline command itself
PROFILE_COUNTER_BENCH = "python3 bench.py --gpus 1 --steps 20 --warmup 5 --no-cpu-baseline --no-extras"


def profile_cmd(workload: str, counters: bool) -> str:
    """The bench command a profile of `workload` runs: the headline command itself for the
    headline's kernel trace, else the same steps without the CPU baseline and the extras."""
    if workload == "high_batch":
        return PROFILE_COUNTER_BENCH if counters else PROFILE_BENCH
    return PROFILE_COUNTER_BENCH + f" --workload {workload}"


def find_workload(name: str):
    """A named workload, or a point of the long-context sweep by its name."""
    import synth
    if name in synth.WORKLOADS:
        return synth.WORKLOADS[name]
    for w in synth.sweep_workloads():
        if w.name == name:
            return w
    raise SystemExit(f"unknown workload {name!r}: one of {sorted(synth.WORKLOADS)} or a sweep point name "
                     "(sweep_s<steps>_k<topk>_d<D>_b<B>_p<p>)")


PREFIX_KERNEL = "tv::k_attn_mfma<4, 1, false>"  # the contiguous-pool instance the benchmark runs
STEP_KERNELS = ("k_tree_mask", "k_scratch", "k_attn_mfma", "k_attn_merge", "k_attn_finish", "k_accept", "k_refresh")
# what one tv_verify_attn call launches (k_attn_merge: split prefixes on the MFMA path;
# k_attn_finish: the vector-ALU path's merge)
CALL_KERNELS = ("k_scratch", "k_attn_mfma", "k_attn_merge", "k_attn_finish")


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def _headline_steps(trace_csv: str, n_steps: int) -> list:
    """The first n_steps steps of the run from a rocprofv3 kernel trace: the library's
    dispatches in start order, cut at each k_tree_mask (a step's first kernel); each step is
    a list of (kernel, start ns, end ns)."""
    import csv
    rows = sorted(((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                   for r in csv.DictReader(open(trace_csv)) if "tv::" in r["Kernel_Name"]), key=lambda x: x[1])
    steps, cur = [], None
    for k, a_, b_ in rows:
        if "k_tree_mask" in k:
            if cur is not None:
                steps.append(cur)
                if len(steps) == n_steps:
                    return steps
            cur = []
        if cur is not None:
            cur.append((k, a_, b_))
    if cur is not None and len(steps) < n_steps:
        steps.append(cur)
    return steps


def _counter_per_kernel(path: str, counter: str) -> dict:
    """Mean value of a counter per dispatch (FETCH_SIZE / WRITE_SIZE: KiB; the derived
    utilisation metrics: percent or a ratio), by kernel name, from a rocprofv3 csv."""
    import csv
    acc = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            v = acc.setdefault(r["Kernel_Name"], [0.0, 0])
            v[0] += float(r["Counter_Value"])
            v[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def summarize_profiles(d: str, workload: str) -> None:
    """Turn the rocprofv3 csv runs of the profiling commands below into the committed
    summaries: every launch of the headline's steps in order (warm-up and timed), the
    tv_verify_attn call's span per step and the HBM fraction that follows from the trace,
    the scaled HBM bytes per call and the traffic record bench.py reports (tagged with the
    digest of the call's kernel sources)."""
    import csv
    out_dir = os.path.join(ROOT, "profiles")
    bench_line = [l for l in open(os.path.join(d, "kt.txt")).read().splitlines() if l.startswith("{")][-1]
    bl = json.loads(bench_line)
    W, K = bl["warmup"], bl["steps"]
    kt_cmd = f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- {profile_cmd(workload, False)}"
    steps = _headline_steps(os.path.join(d, "kt", "run_kernel_trace.csv"), W + K)
    alg = bl["roofline"]["algorithmic_bytes_per_launch"]
    cfg = bl["config"]
    lines = [f"# Kernel trace of the bench command: the verify step at {workload} "
             f"(B={cfg['B']}, D={cfg['D']}, {cfg['Hq']}/{cfg['Hkv']} heads, d={cfg['head_dim']}, {bl['dtype']}, "
             f"{cfg['prefix_tokens']}-token prefix)", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", "    " + kt_cmd, "",
             f"Every launch of the run's {W} untimed and {K} timed steps, in order (`run_kernel_trace.csv`), in us.",
             "`call` is the tv_verify_attn call on the GPU: from the start of its first kernel to the end of its last;",
             "`step` from the step's first kernel start to its last kernel end.", "",
             "| step | " + " | ".join(k.replace("k_", "") for k in STEP_KERNELS) + " | call | step |",
             "|---|" + "---|" * (len(STEP_KERNELS) + 2)]
    calls = []
    for i, st in enumerate(steps):
        dur = {k: 0.0 for k in STEP_KERNELS}
        for name, a_, b_ in st:
            for k in STEP_KERNELS:
                if k + "<" in name or k + "(" in name:
                    dur[k] += (b_ - a_) / 1e3
        vk = [(a_, b_) for name, a_, b_ in st if any(k + "<" in name or k + "(" in name for k in CALL_KERNELS)]
        call = (max(b_ for _, b_ in vk) - min(a_ for a_, _ in vk)) / 1e3 if vk else 0.0
        span = (max(b_ for _, _, b_ in st) - min(a_ for _, a_, _ in st)) / 1e3
        if i >= W:
            calls.append(call)
        lines.append(f"| {i}{'' if i >= W else ' (warm-up)'} | " + " | ".join(f"{dur[k]:.1f}" if dur[k] else "-"
                                                                          for k in STEP_KERNELS)
                     + f" | {call:.1f} | {span:.1f} |")
    mean_call = sum(calls) / max(len(calls), 1)
    lines += ["", f"Timed steps: mean call {mean_call:.1f} us in the trace; {alg / 1e9:.4f} GB algorithmic per call "
              f"-> {alg / (mean_call * 1e-6) / 1e9:.1f} GB/s = {alg / (mean_call * 1e-6) / 1e9 / PEAK_HBM_GBS:.4f} of "
              f"8 TB/s.  The bench line of the same run (HIP events around each call, the profiler attached): "
              f"{bl['roofline']['avg_call_ms'] * 1e3:.1f} us, frac {bl['roofline']['frac']}.", "",
              "Bench line of the profiled run:", "", "    " + bench_line, ""]
    open(os.path.join(out_dir, f"verify_call_{workload}_kernel_trace.md"), "w").write("\n".join(lines))

    fetch = _counter_per_kernel(os.path.join(d, "FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    write = _counter_per_kernel(os.path.join(d, "WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter_per_kernel(os.path.join(d, "copy_FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter_per_kernel(os.path.join(d, "copy_WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_name = [k for k in cf if "copy" in k.lower()][0]
    copy_bytes = int(json.loads([l for l in open(os.path.join(d, "copy_FETCH_SIZE.txt")).read().splitlines()
                                 if l.startswith("{")][-1])["calibrate_copy_bytes"])
    fs = copy_bytes / 1024.0 / cf[copy_name]
    ws = copy_bytes / 1024.0 / cw[copy_name]
    in_call = [k for k in fetch if any(c + "<" in k or c + "(" in k for c in CALL_KERNELS)]
    rd = sum(fetch[k] for k in in_call) * 1024.0 * fs
    wr = sum(write.get(k, 0.0) for k in in_call) * 1024.0 * ws
    # algorithmic bytes of the counter runs themselves
    fl = json.loads([l for l in open(os.path.join(d, "FETCH_SIZE.txt")).read().splitlines() if l.startswith("{")][-1])
    alg_c = fl["roofline"]["algorithmic_bytes_per_launch"]
    cmd = f"rocprofv3 --pmc {{}} --output-format csv -d <dir> -o run -- {profile_cmd(workload, True)}"
    rec = {"kernels": [_short(k) for k in in_call], "workload": workload,
           "command_fetch": cmd.format("FETCH_SIZE"), "command_write": cmd.format("WRITE_SIZE"),
           "command_calibration": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d <dir> -o run -- "
                                  "python3 bench.py --calibrate-copy 1024",
           "fetch_size_kib_per_call": round(sum(fetch[k] for k in in_call), 2),
           "write_size_kib_per_call": round(sum(write.get(k, 0.0) for k in in_call), 2),
           "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_size_kib": round(cf[copy_name], 2),
                                "write_size_kib": round(cw[copy_name], 2), "fetch_scale": round(fs, 5),
                                "write_scale": round(ws, 5)},
           "hbm_bytes_per_launch": int(rd + wr), "hbm_read_bytes_per_launch": int(rd),
           "hbm_write_bytes_per_launch": int(wr), "algorithmic_bytes_per_launch": alg_c,
           "hbm_over_algorithmic": round((rd + wr) / alg_c, 4), "kernel_source_digest": kernel_source_digest()}
    open(os.path.join(out_dir, f"traffic_verify_call_{workload}.json"), "w").write(json.dumps(rec, indent=1) + "\n")
    lines = [f"# HBM bytes per tv_verify_attn call (FETCH_SIZE, WRITE_SIZE): the verify step at {workload}", "",
             "Commands (from the repository root, TMPDIR=/tmp), one counter per run:", "",
             "    " + cmd.format("FETCH_SIZE"), "    " + cmd.format("WRITE_SIZE"),
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python3 bench.py --calibrate-copy 1024",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- python3 bench.py --calibrate-copy 1024",
             "", f"Calibration: a {copy_bytes >> 20} MiB device copy reads FETCH_SIZE = {cf[copy_name]:.1f} KiB and "
             f"WRITE_SIZE = {cw[copy_name]:.1f} KiB per dispatch, so FETCH_SIZE is scaled by {fs:.4f} and "
             f"WRITE_SIZE by {ws:.4f}.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |", "|---|---|---|---|---|"]
    for k in sorted(fetch):
        if "tv::" not in k:
            continue
        lines.append(f"| `{_short(k)}` | {fetch[k]:.1f} | {write.get(k, 0.0):.1f} | "
                     f"{fetch[k] * 1024 * fs / 1e6:.2f} | {write.get(k, 0.0) * 1024 * ws / 1e6:.2f} |")
    lines += ["", f"The tv_verify_attn call ({', '.join('`' + _short(k) + '`' for k in in_call)}): "
              f"{(rd + wr) / 1e9:.4f} GB of HBM traffic per call against {alg_c / 1e9:.4f} GB algorithmic: "
              f"ratio {(rd + wr) / alg_c:.4f}.", ""]
    open(os.path.join(out_dir, f"hbm_bytes_{workload}.md"), "w").write("\n".join(lines))
    util = os.path.join(d, "util", "run_counter_collection.csv")
    if os.path.exists(util):
        summarize_utilisation(util, workload, fl)
    print(json.dumps(rec))


UTIL_METRICS = ("MfmaUtil", "VALUBusy", "LdsUtil", "LdsBankConflict")


def summarize_utilisation(path: str, workload: str, bench_line: dict) -> None:
    """The compute side of the prefix kernel from one rocprofv3 pass of derived metrics
    (rocprofv3's own definitions): MFMA busy cycles per SIMD, VALU busy, LDS busy and LDS
    bank conflicts per access, per kernel, as the committed summary."""
    vals = {m: _counter_per_kernel(path, m) for m in UTIL_METRICS}
    cmd = f"rocprofv3 --pmc {' '.join(UTIL_METRICS)} --output-format csv -d <dir> -o run -- {profile_cmd(workload, True)}"
    kernels = sorted({k for v in vals.values() for k in v if "tv::" in k})
    lines = [f"# Compute-side counters per dispatch: the verify step at {workload}", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", "    " + cmd, "",
             "rocprofv3's derived metrics: MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) *",
             "SIMDs); VALUBusy = 100 * sum(SQ_ACTIVE_INST_VALU) / CUs / max(GRBM_GUI_ACTIVE); LdsUtil = 100 *",
             "sum(SQ_LDS_IDX_ACTIVE) / (max(GRBM_GUI_ACTIVE) * CUs); LdsBankConflict = conflict cycles per",
             "conflict-free LDS cycle.", "",
             "| kernel | MfmaUtil % | VALUBusy % | LdsUtil % | LdsBankConflict |", "|---|---|---|---|---|"]
    for k in kernels:
        lines.append(f"| `{k.split('(')[0].replace('void ', '')}` | " +
                     " | ".join(f"{vals[m].get(k, float('nan')):.3g}" for m in UTIL_METRICS) + " |")
    flops = 4.0 * bench_line["config"]["B"] * bench_line["config"]["Hq"] * bench_line["config"]["D"] * \
        bench_line["config"]["head_dim"] * bench_line["roofline"]["algorithmic_bytes_per_launch"] / \
        (bench_line["config"]["B"] * bench_line["config"]["Hkv"] * bench_line["config"]["head_dim"] * 4.0)
    lines += ["", f"Algorithmic MFMA work of the prefix kernel at this shape: about {flops / 1e12:.3f} TFLOP per launch "
              f"(4 * B * Hq * D * d per committed entry), {flops / (bench_line['roofline']['avg_call_ms'] * 1e-3) / 1e12:.0f} "
              "TFLOP/s at the call time of the same run, against 2500 TFLOP/s dense bf16: the matrix cores are busy "
              "for the share of cycles shown.", ""]
    open(os.path.join(ROOT, "profiles", f"utilisation_{workload}.md"), "w").write("\n".join(lines))


SWEEP_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/b{B} -o run -- "
                   "python3 bench.py --sweep <dir>/b{B}.md --sweep-batches {B} --steps 20 --warmup 5")


STEP_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                  "python3 bench.py --workload {W} --steps 100 --warmup 40 --no-cpu-baseline --no-extras")


def summarize_step_trace(d: str, workload: str) -> None:
    """Per-kernel launch statistics of one workload's steps (rocprofv3 kernel trace of the
    STEP_TRACE_CMD run in d): every kernel of the step with its share of the step, as the
    committed summary."""
    import csv
    line = json.loads([l for l in open(os.path.join(d, "run.txt")).read().splitlines() if l.startswith("{")][-1])
    cfg = line["config"]
    rows = [r for r in csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))) if "tv::" in r["Name"]]
    calls = max(int(r["Calls"]) for r in rows)
    lines = [f"# Kernel-trace summary: the verify step at {workload} (B={cfg['B']}, D={cfg['D']}, "
             f"{cfg['Hq']}/{cfg['Hkv']} heads, d={cfg['head_dim']}, {line['dtype']}, {cfg['prefix_tokens']}-token "
             f"prefix, tree {cfg['tree']})", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", "    " + STEP_TRACE_CMD.format(W=workload), "",
             f"Per-kernel statistics over every step of the run (untimed settling steps, then the timed ones: {calls} "
             "launches of each kernel).  The profiler adds its own overhead per launch;",
             f"the bench line of the same run: {line['ms_per_step'] * 1e3:.1f} us per step, verify launch "
             f"{line['roofline']['avg_call_ms'] * 1e3:.1f} us (HIP events).", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'].split('(')[0].replace('void ', '')}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines.append("")
    open(os.path.join(ROOT, "profiles", f"step_{workload}_kernel_trace.md"), "w").write("\n".join(lines))


def summarize_sweep_traces(d: str) -> None:
    """Per-kernel launch statistics of the sweep's steps at each batch size (one rocprofv3
    run per batch size, every point of that batch size: D 5..8, top-k 1 and 2, p 0.5 and
    0.7, cold and warm), as the committed summary."""
    import csv
    lines = ["# Kernel-trace summary: the verify step at a 131072-token prefix, by batch size", "",
             "64/8 heads, d=128, bf16, 32768 C4 + 1024 C128 entries per sequence; every point of the",
             "long-context sweep at that batch size (D 5..8, top-k 1 and 2, p 0.5 and 0.7; cold and warm",
             "where the state is under 1 GiB), each with its settling and timed steps.  Commands (repository",
             "root, TMPDIR=/tmp), one per batch size B:", "", "    " + SWEEP_TRACE_CMD, "",
             "| B | kernel | calls | average us | min us | max us |", "|---|---|---|---|---|---|"]
    for sub in sorted(os.listdir(d), key=lambda x: int(x[1:]) if x[1:].isdigit() else 0):
        path = os.path.join(d, sub, "run_kernel_stats.csv")
        if not (sub.startswith("b") and sub[1:].isdigit() and os.path.exists(path)):
            continue
        for r in csv.DictReader(open(path)):
            if "tv::" not in r["Name"]:
                continue
            lines.append(f"| {sub[1:]} | `{r['Name'].split('(')[0].replace('void ', '')}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                         f"{float(r['MaxNs']) / 1e3:.1f} |")
    lines.append("")
    open(os.path.join(ROOT, "profiles", "step_long_context_kernel_trace.md"), "w").write("\n".join(lines))


def kernel_source_digest() -> str:
    """Digest of the sources of every kernel a tv_verify_attn call can launch and of the
    host code that plans it."""
    h = hashlib.sha256()
    for f in ("attn_mfma.hip", "scratch_pad.h", "scratch.hip", "attn_merge.hip", "tv_common.h", "tv_host.cpp"):
        with open(os.path.join(ROOT, "tree_speculative_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per tv_verify_attn call from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_verify_call_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def pooled_state(w, caps, draw_seqs=None):
    """Device state of workload w at step 0 with the committed compressed entries drawn
    directly (synth.pooled_prefix); device sequence i holds the workload's sequence
    draw_seqs[i] (default: i)."""
    import concurrent.futures as cf
    import synth
    import tree_speculative_decoding_amd as tv
    seqs = list(range(w.B)) if draw_seqs is None else list(draw_seqs)
    st = tv.DeviceState(len(seqs), w.Hkv, w.d, w.dtype, w.levels, caps)

    def draw(b):
        return [(k, tv.tv.tile_vt(v, st.caps[l])) for l, (k, v) in enumerate(synth.pooled_prefix(w, b))]

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for i, lv in enumerate(ex.map(draw, seqs)):
            for l, (k, vt) in enumerate(lv):
                st.write_seq(l, i, tv.to_device(k, w.dtype), tv.to_device(vt, w.dtype))
                st.n[l][i] = k.shape[1]
    st.P.fill_(w.P)
    return st


class StepRunner:
    """Per-step buffers of one (B, D, Hq) shape and the four calls of one step on `stream`."""

    def __init__(self, w, st, parts: int, stream, in_place: bool = True, deferred: int = 0):
        import torch
        import tree_speculative_decoding_amd as tv
        B, D, Hq, Hkv, d, dev = st.B, w.D, w.Hq, w.Hkv, w.d, "cuda"
        self.w, self.parts, self.stream = w, parts, stream
        self.fused = False  # accept + refresh as one tv_accept_refresh launch
        self.anc = torch.zeros(B, D, dtype=torch.int64, device=dev)
        self.depth = torch.zeros(B, D, dtype=torch.int32, device=dev)
        self.err = torch.zeros(B, dtype=torch.int32, device=dev)
        self.out = torch.zeros(B, D, Hq, d, dtype=tv.tv.torch_dtype(w.dtype), device=dev)
        self.lse = torch.zeros(B, D, Hq, dtype=torch.float32, device=dev)
        self.m = torch.zeros(B, dtype=torch.int32, device=dev)
        self.path = torch.zeros(B, D, dtype=torch.int32, device=dev)
        self.bonus = torch.zeros(B, dtype=torch.int32, device=dev)
        self.log = torch.zeros(B, len(w.levels), D, 2, dtype=torch.int32, device=dev)
        self.sc = tv.DeviceScratch(B, D, Hkv, d, w.dtype, len(w.levels), in_place=in_place, deferred=deferred)
        self.ws = torch.empty(tv.tv_verify_attn_workspace_bytes(D, Hq, st, parts) // 4 + 64, dtype=torch.float32,
                              device=dev)

    def inputs(self, t: int, batch=None) -> dict:
        import torch
        import synth
        import tree_speculative_decoding_amd as tv
        s = synth.step_inputs(self.w, t, batch=batch)
        i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
        return dict(parents=i32(s.parents), draft=i32(s.draft), target=i32(s.target),
                    q=tv.to_device(s.q, self.w.dtype), kt=tv.to_device(s.k_tree, self.w.dtype),
                    vt=tv.to_device(s.v_tree, self.w.dtype))

    def step(self, st, x: dict, attn_ev=None):
        """One step; attn_ev = (start, stop) events recorded on the stream around the whole
        tv_verify_attn call (every kernel it launches)."""
        import tree_speculative_decoding_amd as tv
        s = self.stream
        tv.tv_build_tree_mask(x["parents"], self.anc, self.depth, self.err, s)
        if attn_ev is not None:
            record(attn_ev[0], s)
        tv.tv_verify_attn(x["q"], x["kt"], x["vt"], self.anc, self.depth, self.err, st, self.sc, self.out, self.lse,
                          self.ws, self.parts, s)
        if attn_ev is not None:
            record(attn_ev[1], s)
        if self.fused:
            tv.tv_accept_refresh(st, self.sc, x["parents"], self.anc, self.depth, x["draft"], x["target"], x["kt"],
                                 x["vt"], self.m, self.path, self.bonus, self.log, self.err, s)
            return
        tv.tv_accept(x["parents"], self.anc, self.depth, x["draft"], x["target"], self.err, self.m, self.path,
                     self.bonus, s)
        tv.tv_refresh_state(st, self.sc, x["kt"], x["vt"], self.m, self.path, self.log, self.err, s)


def record(ev: "TimingEvent", stream) -> None:
    if TimingEvent._hip.hipEventRecord(ctypes_ptr(ev.handle), ctypes_ptr(stream.cuda_stream)) != 0:
        raise RuntimeError("hipEventRecord failed")


def settle_warmup(runner: StepRunner, states: list, sets: list, warmup: int, settle_ms: float = 15.0) -> int:
    """Untimed steps to run before timing: at least `warmup`, and enough to keep the GPU
    busy for `settle_ms` (measured launches run up to ~15% slower a few ms into a busy
    period, then settle), from a 3-step estimate of the step time."""
    import torch
    a_, b_ = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    record(a_, runner.stream)
    for t in range(3):
        runner.step(states[t % len(states)], sets[t % len(sets)])
    record(b_, runner.stream)
    torch.cuda.synchronize()
    per = max(a_.elapsed_ms(b_) / 3.0, 1e-3)
    return max(warmup, min(SWEEP_MAX_WARMUP, int(math.ceil(settle_ms / per))))


def timed_steps(runner: StepRunner, states: list, sets: list, warmup: int, steps: int) -> dict:
    """`warmup` untimed steps, then `steps` timed ones, rotating over `states` (so that a
    small working set is read cold from HBM each step) and the input `sets`.  Returns the
    whole region's time, per-step times (fence-free events between steps), the times of
    the tv_verify_attn calls (fence-free events on the stream around each call: every
    kernel the call launches) and the committed lengths before and after the timed steps."""
    import torch
    import tree_speculative_decoding_amd as tv
    stream = runner.stream
    attn_ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    step_ev = [TimingEvent() for _ in range(steps + 1)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the timed steps are queued right behind the warm-up (no host synchronisation and no
    # first-use library kernel in between: an idle GPU restarts the slow first milliseconds)
    for t in range(warmup):
        runner.step(states[t % len(states)], sets[t % len(sets)])
    n_dev = [[x.clone() for x in st.n] for st in states]
    P_before = [st.P.clone() for st in states]
    start.record(stream)
    for t in range(steps):
        record(step_ev[t], stream)
        runner.step(states[(warmup + t) % len(states)], sets[(warmup + t) % len(sets)], attn_ev[t])
    record(step_ev[steps], stream)
    stop.record(stream)
    torch.cuda.synchronize()
    n_before = [sum(int(x.sum()) for x in nd) for nd in n_dev]
    return {"total_ms": start.elapsed_time(stop),
            "step_ms": [step_ev[t].elapsed_ms(step_ev[t + 1]) for t in range(steps)],
            "attn_ms": [a_.elapsed_ms(b_) for a_, b_ in attn_ev],
            "n_before": n_before, "n_after": [sum(int(x.sum()) for x in st.n) for st in states],
            "P_advance": sum(int((st.P - p0).sum()) for st, p0 in zip(states, P_before))}


def attn_bytes_per_launch(w, B: int, entries_per_seq_head: float, tail: float) -> float:
    """Algorithmic bytes of one verify-attention launch: every committed entry's K and V
    once, the raw tail (< C0 tokens), Q in, O out, the tree tokens' K and V, and the plan
    (parents, mask, depth: 16 B per node)."""
    e = 2 if w.dtype == "bf16" else 4
    return B * (w.Hkv * (entries_per_seq_head + tail) * w.d * 2 * e + w.D * w.Hq * w.d * 2 * e
                + w.D * w.Hkv * w.d * 2 * e + 16 * w.D)


def pct(xs, q) -> float:
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the verify path is "
              "implemented and measured on a single GPU (every call is independent per sequence, so "
              "sequences would be split over GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.summarize_sweep_traces:
        summarize_sweep_traces(args.summarize_sweep_traces)
        return
    if args.summarize_step_trace:
        summarize_step_trace(args.summarize_step_trace, args.workload)
        return
    if args.sweep:
        sweep(args)
        return

    import torch

    import synth
    import tree_speculative_decoding_amd as tv

    w = find_workload(args.workload)
    torch.cuda.set_device(0)
    B, D = w.B, w.D
    total_steps = args.warmup + args.steps
    caps = [tv.round_cap(w.P // C + math.ceil(total_steps * D / C) + 2) for C in w.levels]

    # persistent state (committed compressed entries drawn directly) and N_INPUT_SETS
    # per-step input sets, rotated; all resident before timing.  A state under 1 GiB
    # (the small workloads) would be read from the 256 MB last-level cache step after
    # step: ceil(1 GiB / size) + 1 states of different sequences rotate instead, so every
    # step reads its pools from HBM (the warm figure, one state, is reported beside).
    t0 = time.time()
    per_state = B * w.Hkv * sum(caps) * w.d * 2 * (2 if w.dtype == "bf16" else 4)
    n_rot = math.ceil((1 << 30) / per_state) + 1 if per_state < (1 << 30) else 1
    states = [pooled_state(w.with_(B=B * n_rot), caps, range(r * B, (r + 1) * B)) for r in range(n_rot)]
    st = states[0]
    stream = torch.cuda.current_stream()
    deferred = (1 << (len(w.levels) - 1)) if args.defer_coarse and len(w.levels) > 1 else 0
    runner = StepRunner(w, st, args.parts, stream, in_place=not args.no_in_place, deferred=deferred)
    sets = [runner.inputs(t) for t in range(N_INPUT_SETS)]
    saved_all = [snapshot(x) for x in states]
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    r = timed_steps(runner, states, sets, args.warmup, args.steps)
    ms_step = r["total_ms"] / args.steps
    attn_avg_ms = float(np.mean(r["attn_ms"]))
    accepted = r["P_advance"] / B / args.steps  # mean m + 1 per step
    if n_rot > 1:  # the same steps on one state, back to back (its pools partly or wholly cached)
        for x, sv in zip(states, saved_all):
            restore(x, sv)
        rw = timed_steps(runner, [st], sets, args.warmup, args.steps)
        warm = {"ms_per_step": round(rw["total_ms"] / args.steps, 4),
                "attn_ms": round(float(np.mean(rw["attn_ms"])), 5),
                "note": "one state back to back: its pools are read partly or wholly from the last-level cache"}

    # the pools grow during the timed steps: their entries are averaged over the steps
    entries_per_seq_head = (sum(r["n_before"]) + sum(r["n_after"])) / 2.0 / len(states) / B
    tail = float((st.P % w.levels[0]).float().mean().item()) if w.levels[0] > 1 else 0.0
    attn_bytes = attn_bytes_per_launch(w, B, entries_per_seq_head, tail)
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    errs = int((runner.err != 0).sum())

    result = {
        "metric": "verified tree tokens/sec at D=8 bs=64 + achieved HBM GB/s fraction of peak",
        "value": round(B * D / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "D": D, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.d,
                   "prefix_tokens": w.P, "levels": list(w.levels), "tree": w.spec_name,
                   "p_agree": w.p_agree, "prefix_workgroups": args.parts or "auto",
                   "refresh_skip": "off" if args.no_in_place else "in-place chain",
                   "coarse_level": "deferred to the refresh" if deferred else "scratch pad",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w.name),
                     "kernel": "tv_verify_attn call (scratch pad, prefix stream with tail and chain, merge if any)",
                     "avg_call_ms": round(attn_avg_ms, 5),
                     "algorithmic_bytes_per_launch": int(attn_bytes)},
        "step_ms_p10_p50_p90": [round(pct(r["step_ms"], q), 4) for q in (10, 50, 90)],
        **({"warm": warm} if n_rot > 1 else {}),
        "attn_ms_p10_p50_p90": [round(pct(r["attn_ms"], q), 4) for q in (10, 50, 90)],
        "state_bytes": per_state, "rotated_states": n_rot,
        "accepted_length": round(accepted, 4),
        "seq_errors": errs,
        "setup_s": round(setup_s, 1),
    }
    if not args.no_extras:
        # the same steps with acceptance and refresh fused, and both step forms replayed from
        # captured graphs: alternating blocks from the same starting state (A/B in one run)
        ab = ab_blocks(runner, states, sets, args.steps, args.warmup, saved_all)
        result["graph_ms_per_step"] = ab["graph"]
        result["graph_tokens_per_s"] = round(B * D / (ab["graph"] * 1e-3), 1)
        result["fused_accept_refresh"] = {
            "ms_per_step": ab["eager_fused"], "graph_ms_per_step": ab["graph_fused"],
            "graph_tokens_per_s": round(B * D / (ab["graph_fused"] * 1e-3), 1),
            "same_blocks_eager_ms_per_step": ab["eager"],
            "note": "tv_accept_refresh in place of tv_accept + tv_refresh_state; medians of alternating blocks "
                    "(eager, eager fused, graph, graph fused; rotated order) from the same starting state"}
        ceiling = read_ceiling(stream)
        ceiling["attn_frac_of_ceiling"] = round(achieved / ceiling["GB/s"], 4)
        result["read_ceiling"] = ceiling
        result["draft_tree"] = time_draft_tree(w, args.steps, stream)
        result["draft_attn"] = time_draft_attn(w, st, stream, reps=10)
        result["paged_pool"] = time_paged(w, st, stream, reps=5)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def read_ceiling(stream, gib: int = 4) -> dict:
    """The device's practical HBM read ceiling: a plain read-reduce kernel (libtv_measure.so)
    over `gib` GiB, with plain and with nontemporal loads, launched with 2, 4 and 8
    workgroups per CU, 5 timed launches each (fence-free events on `stream`); the best
    average."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "tree_speculative_decoding_amd", "libtv_measure.so"))
    lib.tvm_read_stream.restype = ctypes.c_int
    lib.tvm_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus * 8, dtype=torch.int32, device="cuda")
    best, rows = 0.0, {}
    for nt, per_cu in [(nt, n) for nt in (0, 1) for n in (2, 4, 8)]:
        launch = lambda: lib.tvm_read_stream(buf.data_ptr(), nbytes, cus * per_cu, nt, sink.data_ptr(),
                                             stream.cuda_stream)
        if launch() != 0:
            raise RuntimeError("tvm_read_stream failed")
        ev = [(TimingEvent(), TimingEvent()) for _ in range(5)]
        for a_, b_ in ev:
            record(a_, stream)
            launch()
            record(b_, stream)
        torch.cuda.synchronize()
        gbs = nbytes / (float(np.mean([a_.elapsed_ms(b_) for a_, b_ in ev])) * 1e-3) / 1e9
        rows[f"{per_cu}_per_cu{'_nt' if nt else ''}"] = round(gbs, 1)
        best = max(best, gbs)
    del buf
    torch.cuda.empty_cache()
    return {"GB/s": round(best, 1), "frac_of_peak": round(best / PEAK_HBM_GBS, 4), "bytes": nbytes,
            "by_workgroups": rows, "kernel": "plain read-reduce, 16-byte loads (plain or nontemporal), 8 in flight per thread"}


SWEEP_P = 131072
SWEEP_MAX_WARMUP = 400  # steps; 15 ms at the fastest point (B=1, ~40 us of attention) needs < 400


def sweep(args) -> None:
    """Long-context budget sweep: D in 5..8 x batch in {1, 4, 16, 64} x top-k {1, 2} (k=1:
    a chain of D-1 draft steps; k=2: 3 steps pruned to D), 64/8 heads, d=128, bf16,
    131072-token prefix (32768 C4 + 1024 C128 entries).  Agreement p only changes the
    accepted length, so each (D, B, k) is timed once per p in {0.5, 0.7} with that
    point's own trees and tokens.  The committed state is drawn once per batch size and
    restored before every point; when one state is under 1 GiB, ceil(1 GiB / size) + 1
    states (different sequences) are rotated so every step reads cold from HBM, and the
    same point is also timed warm (one state, back to back), labelled so.  Writes a
    markdown table to args.sweep and prints one JSON line per point."""
    import torch
    import synth
    import tree_speculative_decoding_amd as tv
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    keep = {int(x) for x in args.sweep_batches.split(",") if x}
    points = [w for w in synth.sweep_workloads() if w.B in keep]
    steps, warmup = args.steps, args.warmup
    ceiling = read_ceiling(stream)
    rows = []
    oracle_rows = {}
    for B in sorted({w.B for w in points}):
        ws_ = [w for w in points if w.B == B]
        w0 = ws_[0]
        extra = (steps + max(warmup, SWEEP_MAX_WARMUP)) * max(w.D for w in ws_)
        caps = [tv.round_cap(SWEEP_P // C + math.ceil(extra / C) + 2) for C in w0.levels]
        per_state = B * w0.Hkv * sum(caps) * w0.d * 2 * 2
        n_rot = math.ceil((1 << 30) / per_state) + 1 if per_state < (1 << 30) else 1
        t0 = time.time()
        states = [pooled_state(w0.with_(B=B * n_rot), caps, range(r * B, (r + 1) * B)) for r in range(n_rot)]
        saved = [snapshot(st) for st in states]
        torch.cuda.synchronize()
        print(f"# batch {B}: {n_rot} state(s) of {per_state / 1e9:.3f} GB, {time.time() - t0:.1f} s", file=sys.stderr,
              flush=True)
        for w in ws_:
            runner = StepRunner(w, states[0], 0, stream)
            sets = [runner.inputs(t) for t in range(N_INPUT_SETS)]
            modes = [("cold", states)] if n_rot > 1 else [("hbm", states)]
            if n_rot > 1:
                modes.append(("warm", states[:1]))
            for mode, sts in modes:
                for st, sv in zip(states, saved):
                    restore(st, sv)
                wu = settle_warmup(runner, sts, sets, warmup)
                for st, sv in zip(states, saved):
                    restore(st, sv)
                r = timed_steps(runner, sts, sets, wu, steps)
                ms_step = r["total_ms"] / steps
                attn = float(np.mean(r["attn_ms"]))
                ent = (sum(r["n_before"]) + sum(r["n_after"])) / 2.0 / len(sts) / B
                nbytes = attn_bytes_per_launch(w, B, ent, 0.0)
                gbs = nbytes / (attn * 1e-3) / 1e9
                row = {"point": w.name, "D": w.D, "B": B, "topk": w.topk, "p_agree": w.p_agree, "mode": mode,
                       "intensity_flop_per_byte": round(4.0 * w.Hq * w.D * w.d * ent * B / nbytes, 1),
                       "attn_us": round(attn * 1e3, 1),
                       "attn_us_p10_p50_p90": [round(pct(r["attn_ms"], q) * 1e3, 1) for q in (10, 50, 90)],
                       "attn_GBps": round(gbs, 1), "attn_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                       "attn_frac_of_ceiling": round(gbs / ceiling["GB/s"], 4),
                       "step_us": round(ms_step * 1e3, 1),
                       "step_us_p10_p50_p90": [round(pct(r["step_ms"], q) * 1e3, 1) for q in (10, 50, 90)],
                       "verified_tokens_per_s": round(B * w.D / (ms_step * 1e-3), 1),
                       "accepted_length": round(r["P_advance"] / B / steps, 3),
                       "seq_errors": int((runner.err != 0).sum())}
                if mode != "warm":
                    row["graph_step_us"] = round(graph_step_ms(runner, sts, sets, steps, states, saved) * 1e3, 1)
                    row["graph_verified_tokens_per_s"] = round(B * w.D / (row["graph_step_us"] * 1e-6), 1)
                    runner.fused = True
                    row["graph_fused_step_us"] = round(graph_step_ms(runner, sts, sets, steps, states, saved) * 1e3, 1)
                    runner.fused = False
                rows.append(row)
                print(json.dumps(row), flush=True)
            del runner, sets
        del states, saved
        torch.cuda.empty_cache()
        # the oracle beside the GPU: a time-budgeted sample of this batch size's D = 8, top-k 2
        # point on the host's cores (per-sequence work, so its tokens/s does not depend on B)
        if not args.no_cpu_baseline:
            w8 = [w for w in ws_ if w.D == 8 and w.topk == 2][0]
            ob = cpu_baseline(w8, args.cpu_seconds)
            ob["point"] = w8.name
            oracle_rows[B] = ob
            print(json.dumps({"oracle_B": B, **ob}), flush=True)
    write_sweep_table(args, rows, ceiling, oracle_rows)


def graph_step_ms(runner: StepRunner, sts: list, sets: list, steps: int, states: list, saved: list) -> float:
    """The same steps captured once in a HIP graph (the calls allocate and synchronise
    nothing) and replayed: the step time without host launch overhead.  States are
    restored before the warm-up replay and (queued behind it) before the timed one."""
    import torch
    import tree_speculative_decoding_amd as tv

    def reset():
        for st, sv in zip(states, saved):
            restore(st, sv)
        torch.cuda.synchronize()

    reset()
    g = torch.cuda.CUDAGraph()
    eager_stream = runner.stream
    with torch.cuda.graph(g):
        runner.stream = torch.cuda.current_stream()
        for t in range(steps):
            runner.step(sts[t % len(sts)], sets[t % len(sets)])
    runner.stream = eager_stream
    reset()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    for st, sv in zip(states, saved):  # queued behind the warm replay: no idle gap
        restore(st, sv)
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    del g
    return ms


AB_ROUNDS = 3


def ab_blocks(runner: StepRunner, states: list, sets: list, steps: int, warmup: int, saved: list) -> dict:
    """The four step forms -- eager four calls, eager with tv_accept_refresh, and both
    replayed from a captured HIP graph -- timed in AB_ROUNDS rounds of alternating blocks,
    each block from the same restored starting state (`warmup` untimed steps or one untimed
    replay first), the order rotated every round, all queued without a host
    synchronisation.  Returns the median ms per step of each form."""
    import torch

    def reset():
        for st, sv in zip(states, saved):
            restore(st, sv)

    graphs = {}
    for name, fused in (("graph", False), ("graph_fused", True)):
        reset()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        eager_stream = runner.stream
        runner.fused = fused
        with torch.cuda.graph(g):
            runner.stream = torch.cuda.current_stream()
            for t in range(steps):
                runner.step(states[t % len(states)], sets[t % len(sets)])
        runner.stream = eager_stream
        graphs[name] = g
    runner.fused = False
    stream = runner.stream
    forms = ["eager", "eager_fused", "graph", "graph_fused"]
    ev = {f: [] for f in forms}
    reset()
    torch.cuda.synchronize()
    for r in range(AB_ROUNDS):
        for f in forms[r % 4:] + forms[:r % 4]:
            a_, b_ = TimingEvent(), TimingEvent()
            reset()
            if f.startswith("graph"):
                graphs[f].replay()
                reset()
                record(a_, stream)
                graphs[f].replay()
                record(b_, stream)
            else:
                runner.fused = f == "eager_fused"
                for t in range(warmup):
                    runner.step(states[t % len(states)], sets[t % len(sets)])
                reset()
                record(a_, stream)
                for t in range(steps):
                    runner.step(states[t % len(states)], sets[t % len(sets)])
                record(b_, stream)
                runner.fused = False
            ev[f].append((a_, b_))
    torch.cuda.synchronize()
    out = {f: round(float(np.median([a_.elapsed_ms(b_) / steps for a_, b_ in ev[f]])), 4) for f in forms}
    del graphs
    reset()
    torch.cuda.synchronize()
    return out


def snapshot(st) -> dict:
    """Copies of a state's counts, open sums and tail (what a step changes besides pool
    slots at and beyond n, which are never read until committed again)."""
    c = lambda xs: [x.clone() for x in xs]
    return {"P": st.P.clone(), "n": c(st.n), "open_k": c(st.open_k), "open_v": c(st.open_v),
            "tail": c([t for t in (st.tail_k, st.tail_v) if t is not None])}


def restore(st, sv: dict) -> None:
    st.P.copy_(sv["P"])
    for dst, src in zip(st.n + st.open_k + st.open_v, sv["n"] + sv["open_k"] + sv["open_v"]):
        dst.copy_(src)
    for dst, src in zip([t for t in (st.tail_k, st.tail_v) if t is not None], sv["tail"]):
        dst.copy_(src)


def write_sweep_table(args, rows: list, ceiling: dict, oracle_rows: dict) -> None:
    hdr = ["# Long-context budget sweep: verify step at a 131072-token prefix", "",
           "64/8 heads, d=128, bf16, 32768 C4 + 1024 C128 committed entries per sequence; one step = plan,",
           "verify attention with the scratch pad, accept, refresh.  Command (repository root):", "",
           f"    python3 bench.py --sweep <out.md> --steps {args.steps} --warmup {args.warmup}", "",
           f"Read ceiling on the same device (plain read-reduce, 4 GiB): {ceiling['GB/s']:.0f} GB/s "
           f"({100 * ceiling['frac_of_peak']:.1f}% of 8 TB/s).  `cold`: states rotated so each step reads "
           "its pools from HBM; `warm`: one state back to back (batch 1 and 4 fit the 256 MB last-level "
           "cache partly or wholly); `hbm`: one state larger than 1 GiB.  Every point first runs untimed "
           "steps for at least 15 ms.  Attention = the tv_verify_attn call (every kernel it launches: the "
           "scratch pad when it runs apart, the prefix stream, the merge of split prefixes), mean over the timed "
           "steps, p10 / p90 beside it; intensity = "
           "attention flops per algorithmic byte; graph = the same steps replayed from one captured HIP "
           "graph; graph fused = the same with tv_accept_refresh in place of tv_accept + tv_refresh_state.", "",
           "| D | B | top-k | p | mode | intensity | attn us (p10-p90) | attn GB/s | % of 8 TB/s | % of ceiling "
           "| step us | verified tok/s | graph step us | graph tok/s | graph fused step us | accepted length "
           "| oracle tok/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    body = []
    for r in sorted(rows, key=lambda r: (r["B"], r["D"], r["topk"], r["p_agree"], r["mode"])):
        p10, _, p90 = r["attn_us_p10_p50_p90"]
        body.append(f"| {r['D']} | {r['B']} | {r['topk']} | {r['p_agree']} | {r['mode']} | "
                    f"{r['intensity_flop_per_byte']} | {r['attn_us']} ({p10}-{p90}) | {r['attn_GBps']:.0f} | "
                    f"{100 * r['attn_frac_of_peak']:.1f} | {100 * r['attn_frac_of_ceiling']:.1f} | {r['step_us']} | "
                    f"{r['verified_tokens_per_s']:.0f} | {r.get('graph_step_us', '-')} | "
                    f"{r.get('graph_verified_tokens_per_s', '-')} | {r.get('graph_fused_step_us', '-')} | "
                    f"{r['accepted_length']} | {oracle_rows[r['B']]['value'] if r['B'] in oracle_rows else '-'} |")
    foot = ["", "Oracle (the fp64 CPU definition, as it stands) beside the GPU, same run, same host: per batch "
            "size, whole sequences of its D = 8, top-k 2, p = 0.5 point until the time budget is spent "
            "(one full step each; the oracle's work is per sequence, so its tokens/s does not depend on B):", ""]
    for B, ob in sorted(oracle_rows.items()):
        foot.append(f"- B = {B}: {ob['value']} tokens/s on {ob['cores']} cores ({ob['blas']} BLAS, "
                    f"{ob['blas_threads']} threads); {ob['sample']}")
    with open(args.sweep, "w") as fh:
        fh.write("\n".join(hdr + body + (foot if oracle_rows else [])) + "\n")


def time_draft_tree(w, steps: int, stream) -> dict:
    """Device draft-tree construction for the workload's batch and tree shape (top-k,
    draft steps, budget D; vocabulary w.vocab) from synthetic Gumbel draft logits: the
    average of `steps` launches, each timed with fence-free HIP events on `stream`."""
    import torch
    import tree_speculative_decoding_amd as tv
    E = sum(w.topk ** l for l in range(w.steps))
    rng = np.random.default_rng(w.seed + 77)
    logits = torch.from_numpy(rng.gumbel(size=(w.B, E, w.vocab)).astype(np.float32)).cuda()
    root = torch.from_numpy(rng.integers(w.vocab, size=w.B).astype(np.int32)).cuda()
    par = torch.zeros(w.B, w.D, dtype=torch.int32, device="cuda")
    tok = torch.zeros(w.B, w.D, dtype=torch.int32, device="cuda")
    tv.tv_build_draft_tree(logits, root, w.topk, w.steps, par, tok, stream=stream)  # warm-up
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    hip = TimingEvent._hip
    for a_, b_ in ev:
        hip.hipEventRecord(ctypes_ptr(a_.handle), ctypes_ptr(stream.cuda_stream))
        tv.tv_build_draft_tree(logits, root, w.topk, w.steps, par, tok, stream=stream)
        hip.hipEventRecord(ctypes_ptr(b_.handle), ctypes_ptr(stream.cuda_stream))
    torch.cuda.synchronize()
    us = float(np.mean([a_.elapsed_ms(b_) for a_, b_ in ev])) * 1e3
    return {"us_per_launch": round(us, 2), "B": w.B, "topk": w.topk, "draft_steps": w.steps, "D": w.D,
            "vocab": w.vocab, "logits_bytes": w.B * E * w.vocab * 4,
            "bound": "latency (one workgroup per sequence; E rows of the vocabulary each)"}


DRAFT_WARM_LAUNCHES = 40  # untimed launches ahead of the draft-attention and paged timings
PAGED_ROUNDS = 4


def time_draft_attn(w, st, stream, reps: int) -> dict:
    """Draft-decode reuse of the branch-aware attention: for each level t of the
    workload's expansion (top-k, draft steps), tv_draft_attn over the 1 + k + ... +
    k^(t-1) nodes created so far, with one plan of the whole expansion shared by the
    levels; after DRAFT_WARM_LAUNCHES untimed launches, `reps` launches back to back, each
    timed with fence-free events on `stream`.  Synthetic Q / tree K/V of the workload's
    dtype; the state is the benchmark's."""
    import torch
    import synth
    import tree_speculative_decoding_amd as tv
    k, s = w.topk, w.steps
    n = sum(k ** l for l in range(s + 1))
    rng = np.random.default_rng(w.seed + 78)
    par = np.array([-1] + [(c - 1) // k for c in range(1, n)], dtype=np.int32)
    parents = torch.from_numpy(np.tile(par, (w.B, 1))).cuda()

    def vals(shape):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        return tv.to_device(synth.f32_to_bf16_bits(x) if w.dtype == "bf16" else x, w.dtype)

    q, kt, vt = vals((w.B, n, w.Hq, w.d)), vals((w.B, n, w.Hkv, w.d)), vals((w.B, n, w.Hkv, w.d))
    anc = torch.zeros(w.B, n, dtype=torch.int64, device="cuda")
    depth = torch.zeros(w.B, n, dtype=torch.int32, device="cuda")
    err = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    tv.tv_build_tree_mask(parents, anc, depth, err, stream)
    e = 2 if w.dtype == "bf16" else 4
    entries = sum(int(x.sum()) for x in st.n) / w.B
    tail = float((st.P % w.levels[0]).float().mean().item()) if w.levels[0] > 1 else 0.0
    levels, us, frac = [], [], []
    for t in range(1, s + 1):
        D = sum(k ** l for l in range(t))
        qd, kd, vd = q[:, :D].contiguous(), kt[:, :D].contiguous(), vt[:, :D].contiguous()
        out = torch.empty(w.B, D, w.Hq, w.d, dtype=qd.dtype, device="cuda")
        ws = torch.empty(tv.tv_verify_attn_workspace_bytes(D, w.Hq, st) // 4 + 64, dtype=torch.float32,
                         device="cuda")
        # untimed launches first (the clock settles ~10 ms into a busy period), then the
        # timed ones queued right behind them
        for _ in range(DRAFT_WARM_LAUNCHES):
            tv.tv_draft_attn(qd, kd, vd, anc, err, st, out, None, ws, stream=stream)
        ev = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        for a_, b_ in ev:
            record(a_, stream)
            tv.tv_draft_attn(qd, kd, vd, anc, err, st, out, None, ws, stream=stream)
            record(b_, stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a_.elapsed_ms(b_) for a_, b_ in ev]))
        nbytes = w.B * (w.Hkv * (entries + tail) * w.d * 2 * e + D * w.Hq * w.d * 2 * e + D * w.Hkv * w.d * 2 * e
                        + 8 * D)
        levels.append(D)
        us.append(round(ms * 1e3, 1))
        frac.append(round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    return {"nodes_per_level": levels, "us_per_launch": us, "hbm_frac": frac, "expansion_nodes": n,
            "note": "same prefix stream as verify; rows for every node created so far"}


def time_paged(w, st, stream, reps: int) -> dict:
    """Gather cost of a paged pool: the benchmark's state copied into 64-entry pages at
    random physical positions; after untimed launches, PAGED_ROUNDS rounds of `reps`
    back-to-back verify launches on the contiguous and then the paged state (same inputs,
    no refresh, so both stay equal)."""
    import torch
    import synth
    import tree_speculative_decoding_amd as tv
    A = 64
    sp = tv.DeviceState(w.B, w.Hkv, w.d, w.dtype, w.levels, st.caps, page_seed=w.seed + 79)
    for l in range(len(w.levels)):
        pps = st.caps[l] // A
        pages = sp.page_table[l].long().reshape(-1)
        sp.pool_k[l][pages] = (st.logical_k(l).reshape(w.B, w.Hkv, pps, A, w.d).permute(0, 2, 1, 3, 4)
                               .reshape(w.B * pps, w.Hkv, A, w.d))
        sp.pool_vt[l][pages] = st.logical_vt(l).permute(0, 2, 1, 3, 4).reshape(w.B * pps, w.Hkv, w.d, A)
        sp.n[l].copy_(st.n[l])
        sp.open_k[l].copy_(st.open_k[l])
        sp.open_v[l].copy_(st.open_v[l])
    if st.tail_k is not None:
        sp.tail_k.copy_(st.tail_k)
        sp.tail_v.copy_(st.tail_v)
    sp.P.copy_(st.P)
    s = synth.step_inputs(w, 0)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    q, kt, vt = tv.to_device(s.q, w.dtype), tv.to_device(s.k_tree, w.dtype), tv.to_device(s.v_tree, w.dtype)
    anc = torch.zeros(w.B, w.D, dtype=torch.int64, device="cuda")
    depth = torch.zeros(w.B, w.D, dtype=torch.int32, device="cuda")
    err = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    tv.tv_build_tree_mask(i32(s.parents), anc, depth, err, stream)
    out = [torch.empty(w.B, w.D, w.Hq, w.d, dtype=q.dtype, device="cuda") for _ in range(2)]
    ws = torch.empty(tv.tv_verify_attn_workspace_bytes(w.D, w.Hq, st) // 4 + 64, dtype=torch.float32, device="cuda")
    # untimed launches first, then blocks of `reps` back-to-back launches of each state,
    # alternating, all queued without a synchronisation in between
    for _ in range(DRAFT_WARM_LAUNCHES):
        tv.tv_verify_attn(q, kt, vt, anc, depth, err, st, None, out[0], None, ws, 0, stream)
    ev = {0: [], 1: []}
    for _ in range(PAGED_ROUNDS):
        for which, state in ((0, st), (1, sp)):
            for _ in range(reps):
                a_, b_ = TimingEvent(), TimingEvent()
                record(a_, stream)
                tv.tv_verify_attn(q, kt, vt, anc, depth, err, state, None, out[which], None, ws, 0, stream)
                record(b_, stream)
                ev[which].append((a_, b_))
    torch.cuda.synchronize()
    ms = {k: [a_.elapsed_ms(b_) for a_, b_ in v] for k, v in ev.items()}
    same = bool(torch.equal(out[0].view(torch.int16), out[1].view(torch.int16))) if w.dtype == "bf16" else \
        bool(torch.equal(out[0], out[1]))
    c, p_ = float(np.mean(ms[0])) * 1e3, float(np.mean(ms[1])) * 1e3
    return {"contiguous_us": round(c, 1), "paged_us": round(p_, 1), "paged_over_contiguous": round(p_ / c, 4),
            "page_entries": A, "outputs_bit_identical": same}


def ctypes_ptr(x):
    import ctypes
    return ctypes.c_void_p(x)


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle, as it stands, on whole sequences of the same workload until the
    time budget is spent (at least one); tokens/s = sequences * D / time."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({str(i.get("internal_api")) for i in info if i.get("user_api") == "blas"})) or "none"
    except Exception:
        threads, blas = 1, "unknown"
    cores = len(os.sched_getaffinity(0))
    caps = [w.P // C + 64 for C in w.levels]
    done, t_used = 0, 0.0
    b = 0
    while done == 0 or t_used < budget_s:
        if b >= w.B:
            break
        ents = [[(oracle.widen(k, w.dtype), oracle.widen(v, w.dtype)) for k, v in synth.pooled_prefix(w, b)]]
        ost = oracle.from_entries(ents, [w.P], w.levels, caps, w.d)
        s = synth.step_inputs(w, 0, batch=[b])
        q, kt, vt = (oracle.widen(a, w.dtype) for a in (s.q, s.k_tree, s.v_tree))
        t0 = time.perf_counter()
        oracle.step(ost, s.parents, s.draft, s.target, q, kt, vt)
        t_used += time.perf_counter() - t0
        done += 1
        b += 1
    return {"value": round(done * w.D / t_used, 2), "unit": "tokens/s", "cores": cores, "blas_threads": threads,
            "kind": "oracle", "blas": blas,
            "sample": f"{done} of {w.B} sequences of {w.name}, one full step each (plan, attention, scratch, "
                      f"accept, refresh), fp64 numpy; input widening excluded; {t_used:.1f} s"}


if __name__ == "__main__":
    main()
