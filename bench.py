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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="high_batch")
    ap.add_argument("--parts", type=int, default=0, help="prefix-stream workgroups (0 = library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the draft-tree, draft-attention and paged-pool measurements (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="time budget of the oracle sample")
    ap.add_argument("--summarize-profiles", default="", metavar="DIR",
                    help="write profiles/*.md and the traffic JSON from rocprofv3 csv runs in DIR "
                         "(kt/, FETCH_SIZE/, WRITE_SIZE/, copy_FETCH_SIZE/, copy_WRITE_SIZE/, kt.txt)")
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
        if TimingEvent._hip is not None and self.handle:
            TimingEvent._hip.hipEventDestroy(self._ct.c_void_p(self.handle))


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


PROFILE_BENCH = "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-extras"
PROFILE_COUNTER_BENCH = "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extras"
PREFIX_KERNEL = "tv::k_attn_mfma<4, 1, false>"  # the contiguous-pool instance the benchmark runs


def _counter_per_kernel(path: str, counter: str) -> dict:
    """Mean counter value (KiB) per dispatch, by kernel name, from a rocprofv3 csv."""
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
    summaries: the kernel-trace statistics, the scaled HBM bytes per dispatch and the
    traffic record bench.py reports (tagged with the prefix kernel's source digest)."""
    import csv
    out_dir = os.path.join(ROOT, "profiles")
    bench_line = [l for l in open(os.path.join(d, "kt.txt")).read().splitlines() if l.startswith("{")][-1]
    bl = json.loads(bench_line)
    kt_cmd = f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- {PROFILE_BENCH}"
    rows = list(csv.DictReader(open(os.path.join(d, "kt", "run_kernel_stats.csv"))))
    ours = [r for r in rows if "tv::" in r["Name"]]
    total_ns = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# Kernel-trace summary: the verify step at {workload} "
             f"(B={bl['config']['B']}, D={bl['config']['D']}, {bl['config']['Hq']}/{bl['config']['Hkv']} heads, "
             f"d={bl['config']['head_dim']}, {bl['dtype']}, {bl['config']['prefix_tokens']}-token prefix)", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", "    " + kt_cmd, "",
             "Per-kernel statistics (`run_kernel_stats.csv`; calls = warm-up + timed steps).  The bench line of",
             f"the same run reports the prefix kernel at avg {bl['roofline']['avg_launch_ms'] * 1e3:.1f} us from HIP "
             f"events on its stream ({bl['roofline']['achieved']:.1f} GB/s).  The profiler slows the kernel; a run",
             "of the same command without it (`python bench.py`) is the throughput figure.", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in ours:
        lines.append(f"| `{r['Name'].split('(')[0].replace('void ', '')}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100.0 * float(r['TotalDurationNs']) / total_ns:.1f}% |")
    lines += ["", "Bench line of the profiled run:", "", "    " + bench_line, ""]
    open(os.path.join(out_dir, f"attn_prefix_{workload}_kernel_trace.md"), "w").write("\n".join(lines))

    fetch = _counter_per_kernel(os.path.join(d, "FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    write = _counter_per_kernel(os.path.join(d, "WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter_per_kernel(os.path.join(d, "copy_FETCH_SIZE", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter_per_kernel(os.path.join(d, "copy_WRITE_SIZE", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_name = [k for k in cf if "copy" in k.lower()][0]
    copy_bytes = int(json.loads([l for l in open(os.path.join(d, "copy_FETCH_SIZE.txt")).read().splitlines()
                                 if l.startswith("{")][-1])["calibrate_copy_bytes"])
    fs = copy_bytes / 1024.0 / cf[copy_name]
    ws = copy_bytes / 1024.0 / cw[copy_name]
    pk = [k for k in fetch if PREFIX_KERNEL in k][0]
    rd = fetch[pk] * 1024.0 * fs
    wr = write[pk] * 1024.0 * ws
    alg = bl["roofline"]["algorithmic_bytes_per_launch"]
    cmd = f"rocprofv3 --pmc {{}} --output-format csv -d <dir> -o run -- {PROFILE_COUNTER_BENCH}"
    rec = {"kernel": pk, "workload": workload,
           "command_fetch": cmd.format("FETCH_SIZE"), "command_write": cmd.format("WRITE_SIZE"),
           "command_calibration": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d <dir> -o run -- "
                                  "python3 bench.py --calibrate-copy 1024",
           "fetch_size_kib_per_dispatch": round(fetch[pk], 2), "write_size_kib_per_dispatch": round(write[pk], 2),
           "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_size_kib": round(cf[copy_name], 2),
                                "write_size_kib": round(cw[copy_name], 2), "fetch_scale": round(fs, 5),
                                "write_scale": round(ws, 5)},
           "hbm_bytes_per_launch": int(rd + wr), "hbm_read_bytes_per_launch": int(rd),
           "hbm_write_bytes_per_launch": int(wr), "algorithmic_bytes_per_launch": alg,
           "hbm_over_algorithmic": round((rd + wr) / alg, 4), "kernel_source_digest": kernel_source_digest()}
    open(os.path.join(out_dir, f"traffic_attn_prefix_{workload}.json"), "w").write(json.dumps(rec, indent=1) + "\n")
    lines = [f"# HBM bytes per dispatch (FETCH_SIZE, WRITE_SIZE): the verify step at {workload}", "",
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
        lines.append(f"| `{k.split('(')[0].replace('void ', '')}` | {fetch[k]:.1f} | {write.get(k, 0.0):.1f} | "
                     f"{fetch[k] * 1024 * fs / 1e6:.2f} | {write.get(k, 0.0) * 1024 * ws / 1e6:.2f} |")
    lines += ["", f"Prefix kernel: {(rd + wr) / 1e9:.4f} GB of HBM traffic per launch against {alg / 1e9:.4f} GB "
              f"algorithmic: ratio {(rd + wr) / alg:.4f}.", ""]
    open(os.path.join(out_dir, f"hbm_bytes_{workload}.md"), "w").write("\n".join(lines))
    print(json.dumps(rec))


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("attn_mfma.hip", "tv_common.h"):
        with open(os.path.join(ROOT, "tree_speculative_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the prefix kernel from committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_attn_prefix_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is single-GPU "
              "in this build.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return

    import torch

    import synth
    import tree_speculative_decoding_amd as tv

    w = synth.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    B, D, Hq, Hkv, d = w.B, w.D, w.Hq, w.Hkv, w.d
    e = 2 if w.dtype == "bf16" else 4
    total_steps = args.warmup + args.steps
    caps = [tv.round_cap(w.P // C + math.ceil(total_steps * D / C) + 2) for C in w.levels]

    # ---- persistent state: committed compressed entries drawn directly (pooled prefix)
    t0 = time.time()
    st = tv.DeviceState(B, Hkv, d, w.dtype, w.levels, caps)
    import concurrent.futures as cf

    def draw(b):
        return [(k, tv.tv.tile_vt(v, st.caps[l])) for l, (k, v) in enumerate(synth.pooled_prefix(w, b))]

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for b, lv in enumerate(ex.map(draw, range(B))):
            for l, (k, vt) in enumerate(lv):
                st.write_seq(l, b, tv.to_device(k, w.dtype), tv.to_device(vt, w.dtype))
                st.n[l][b] = k.shape[1]
    st.P.fill_(w.P)

    # ---- per-step inputs (N_INPUT_SETS sets, rotated)
    sets = []
    for t in range(N_INPUT_SETS):
        s = synth.step_inputs(w, t)
        i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)
        sets.append(dict(parents=i32(s.parents), draft=i32(s.draft), target=i32(s.target),
                         q=tv.to_device(s.q, w.dtype), kt=tv.to_device(s.k_tree, w.dtype),
                         vt=tv.to_device(s.v_tree, w.dtype)))
    anc = torch.zeros(B, D, dtype=torch.int64, device=dev)
    depth = torch.zeros(B, D, dtype=torch.int32, device=dev)
    err = torch.zeros(B, dtype=torch.int32, device=dev)
    out = torch.zeros(B, D, Hq, d, dtype=tv.tv.torch_dtype(w.dtype), device=dev)
    lse = torch.zeros(B, D, Hq, dtype=torch.float32, device=dev)
    m = torch.zeros(B, dtype=torch.int32, device=dev)
    path = torch.zeros(B, D, dtype=torch.int32, device=dev)
    bonus = torch.zeros(B, dtype=torch.int32, device=dev)
    log = torch.zeros(B, len(w.levels), D, 2, dtype=torch.int32, device=dev)
    sc = tv.DeviceScratch(B, D, Hkv, d, w.dtype, len(w.levels))
    ws_bytes = tv.tv_verify_attn_workspace_bytes(D, Hq, st, args.parts)
    ws = torch.empty(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def one_step(x):
        tv.tv_build_tree_mask(x["parents"], anc, depth, err, stream)
        tv.tv_verify_attn(x["q"], x["kt"], x["vt"], anc, depth, err, st, sc, out, lse, ws, args.parts, stream)
        tv.tv_accept(x["parents"], anc, depth, x["draft"], x["target"], err, m, path, bonus, stream)
        tv.tv_refresh_state(st, sc, x["kt"], x["vt"], m, path, log, err, stream)

    for t in range(args.warmup):
        one_step(sets[t % N_INPUT_SETS])
    torch.cuda.synchronize()

    # per-launch events around the prefix kernel (recorded by the library on `stream`)
    ev = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    n_sum_before = sum(int(x.sum()) for x in st.n)
    P_before = st.P.clone()
    acc_len = torch.zeros(B, dtype=torch.int64, device=dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for t in range(args.steps):
        tv.tv_set_timing_events(ev[t][0], ev[t][1])
        one_step(sets[(args.warmup + t) % N_INPUT_SETS])
    stop.record(stream)
    tv.tv_set_timing_events(None, None)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    attn_ms = [a_.elapsed_ms(b_) for a_, b_ in ev]
    attn_avg_ms = float(np.mean(attn_ms))
    n_sum_after = sum(int(x.sum()) for x in st.n)
    accepted = (st.P - P_before).double().mean().item() / args.steps  # mean m + 1 per step

    # Algorithmic bytes of the attention kernel per launch: every committed entry's K and
    # V once (averaged over the timed steps as the pools grow), the raw tail (< C0
    # tokens), Q in, O out, the tree tokens' K and V, and the plan (parents, mask, depth:
    # 16 B per node).  The prefix kernel reads all of these and writes every output row
    # itself when each (sequence, head) prefix is one workgroup's whole slice.
    entries_per_seq_head = (n_sum_before + n_sum_after) / 2.0 / B
    tail = float((P_before % w.levels[0]).float().mean().item()) if w.levels[0] > 1 else 0.0
    attn_bytes = B * (Hkv * (entries_per_seq_head + tail) * d * 2 * e + D * Hq * d * 2 * e
                      + D * Hkv * d * 2 * e + 16 * D)
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    errs = int((err != 0).sum())

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
        "config": {"workload": w.name, "B": B, "D": D, "Hq": Hq, "Hkv": Hkv, "head_dim": d,
                   "prefix_tokens": w.P, "levels": list(w.levels), "tree": w.spec_name,
                   "p_agree": w.p_agree, "prefix_workgroups": args.parts or "auto",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w.name),
                     "kernel": "k_attn_mfma (prefix stream + tail + chain)", "avg_launch_ms": round(attn_avg_ms, 5),
                     "algorithmic_bytes_per_launch": int(attn_bytes)},
        "accepted_length": round(accepted, 4),
        "seq_errors": errs,
        "setup_s": round(setup_s, 1),
    }
    if not args.no_extras:
        result["draft_tree"] = time_draft_tree(w, args.steps, stream)
        result["draft_attn"] = time_draft_attn(w, st, stream, reps=3)
        result["paged_pool"] = time_paged(w, st, stream, reps=5)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


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


def time_draft_attn(w, st, stream, reps: int) -> dict:
    """Draft-decode reuse of the branch-aware attention: for each level t of the
    workload's expansion (top-k, draft steps), tv_draft_attn over the 1 + k + ... +
    k^(t-1) nodes created so far, with one plan of the whole expansion shared by the
    levels; each launch is timed with fence-free events on `stream` (`reps` per level).
    Synthetic Q / tree K/V of the workload's dtype; the state is the benchmark's."""
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
        tv.tv_draft_attn(qd, kd, vd, anc, err, st, out, None, ws, stream=stream)  # warm-up
        ev = [(TimingEvent(), TimingEvent()) for _ in range(reps)]
        for a_, b_ in ev:
            tv.tv_set_timing_events(a_, b_)
            tv.tv_draft_attn(qd, kd, vd, anc, err, st, out, None, ws, stream=stream)
        tv.tv_set_timing_events(None, None)
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
    random physical positions, then `reps` verify launches on each of the contiguous and
    the paged state, alternating (same inputs, no refresh, so both stay equal)."""
    import torch
    import synth
    import tree_speculative_decoding_amd as tv
    A = 64
    sp = tv.DeviceState(w.B, w.Hkv, w.d, w.dtype, w.levels, st.caps, page_seed=w.seed + 79)
    for l in range(len(w.levels)):
        pps = st.caps[l] // A
        pages = sp.page_table[l].long().reshape(-1)
        sp.pool_k[l][pages] = (st.pool_k[l].reshape(w.B, w.Hkv, pps, A, w.d).permute(0, 2, 1, 3, 4)
                               .reshape(w.B * pps, w.Hkv, A, w.d))
        sp.pool_vt[l][pages] = st.pool_vt[l].permute(0, 2, 1, 3, 4).reshape(w.B * pps, w.Hkv, w.d, A)
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
    ms = {0: [], 1: []}
    for i in range(reps + 1):
        for which, state in ((0, st), (1, sp)):
            a_, b_ = TimingEvent(), TimingEvent()
            tv.tv_set_timing_events(a_, b_)
            tv.tv_verify_attn(q, kt, vt, anc, depth, err, state, None, out[which], None, ws, 0, stream)
            tv.tv_set_timing_events(None, None)
            torch.cuda.synchronize()
            if i > 0:  # the first round warms up
                ms[which].append(a_.elapsed_ms(b_))
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
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
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
    return {"value": round(done * w.D / t_used, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.B} sequences of {w.name}, one full step each (plan, attention, scratch, "
                      f"accept, refresh), fp64 numpy; input widening excluded; {t_used:.1f} s"}


if __name__ == "__main__":
    main()
