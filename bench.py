#!/usr/bin/env python3
"""Benchmark of the context-parallel causal attention hot path on one MI355X.

Headline (``value``): causal prefill attention TFLOP/s (unmasked FLOPs only:
4 * D * Hq per visible (query, key) pair) on the 128K-token workload --
1 x 131072 tokens, 16 query heads on 1 KV head, head_dim 128, bf16, seed 3,
cut into 16 CP chunks of 8192 and run in Pass-KV ring order.  One step is one
full ring: 16 ring-step launches (all simulated ranks' pairs of a step in one
launch), each pair's partial (O, LSE) merged into its owner's running result
in the launch's epilogue.  Inputs are resident in HBM before timing starts.

The same JSON line carries the dominant kernel's roofline (HIP events around
every ring-step launch, on the stream the library launches on), the Pass-Q
ring, the ring with per-pair partials and a merge pass, the fused prefill, the
8K-token GQA workload, 2048 new tokens against a 128K cached context (ring
order chosen by exchanged bytes), the split-KV decode (with its
allocation-free form), the KV-cache shard write and decode over the shards,
the 1M-token workload, and the fp64 CPU oracle timed on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-1m]
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR [CLOCK_DIR [SQ_DIR [RDREQ_DIR]]]
  python bench.py --summarize-trace TRACE_DIR BENCH_JSON
"""
from __future__ import annotations

import argparse
import glob
import csv
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 FLOP/clk x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0       # HBM3E
METRIC = "causal prefill attention TFLOP/s & % bf16 MFMA peak; decode GB/s & % HBM peak"
PREFILL = "prefill_bf16_s128k_p16"
DECODE = "decode_b128_kv32k_p8"
KERNEL_SRC = os.path.join(ROOT, "context_attention_cpattn_amd", "csrc", "partial_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_bf16_prefill_s128k_p16_traffic.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "partial_bf16_prefill_s128k_p16_trace.txt")
DECODE_FILE = os.path.join(ROOT, "profiles", "decode_stream_b128_kv32k_p8.txt")
DECODE_PROFILE_CMD = "python $R/bench.py --decode-only"
MERGE_FILE = os.path.join(ROOT, "profiles", "ring_merge_s128k_p16.txt")
MERGE_PROFILE_CMD = "python $R/bench.py --merge-only"
PROFILE_CMD = "python $R/bench.py --headline-only --no-cpu-baseline"
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in ("partial_bf16.hip", "decode.hip", "merge.hip", "device.h", "internal.h"):
        with open(os.path.join(ROOT, "context_attention_cpattn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def ring_step_flops(w, order: str):
    """Unmasked FLOPs of each ring step: 4*D*Hq*B per visible (query, key) pair."""
    P, C = w.n_chunks, w.chunk
    per_pair = 4.0 * w.D * w.Hq * w.B
    out = []
    for s in range(P):
        f = 0.0
        for r in range(P):
            other = (r - s) % P
            qi, kj = (r, other) if order == "pass_kv" else (other, r)
            if w.causal and kj > qi:
                continue
            f += per_pair * (C * (C + 1) / 2 if (w.causal and kj == qi) else C * C)
        out.append(f)
    return out


def _summary_values(path: str, keep_text=()) -> dict:
    """Entries of a committed profile summary (numbers, plus the text keys named); empty if the file
    is absent or a kernel source changed since it was taken."""
    if not os.path.exists(path):
        return {}
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            a, b = ln.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash():
        return {}
    out = {}
    for key, val in kv.items():
        if key in keep_text:
            out[key] = val
            continue
        try:
            out[key] = float(val.split()[0])
        except (ValueError, IndexError):
            pass
    return out


def pmc_values() -> dict:
    """Numeric entries of the committed counter summary of the current kernel sources."""
    return _summary_values(TRAFFIC_FILE)


def trace_values() -> dict:
    """Entries of the committed kernel-trace summary of the current kernel sources."""
    return _summary_values(TRACE_FILE, keep_text=("machine_host", "machine_gpu_uuid"))


def read_pmc_summary():
    """(HBM bytes per launch, shader clock GHz, MFMA busy fraction, fraction of peak at that clock)
    of the partial kernel from the committed pmc summary, each None when unavailable."""
    kv = pmc_values()
    return (kv.get("hbm_bytes_per_launch"), kv.get("sclk_ghz_partial_kernel"), kv.get("mfma_busy_fraction"),
            kv.get("frac_of_peak_at_measured_sclk"))


def cpu_threads() -> int:
    """Host threads for the oracle: every core this process may run on, capped by OMP_NUM_THREADS
    when it is set (the host's CPU share for this job)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(w, q, k, v, seconds: float):
    """The fp64 oracle (``oracle.partial_attention``, as the parity tests call it) on blocks of 256
    consecutive query rows at the end of the prefill workload, each against its full causal
    context, for about ``seconds``: GEMM-shaped row blocks on the host cores."""
    import torch

    import oracle

    threads = cpu_threads()
    torch.set_num_threads(threads)
    R = 256
    S = w.Sq
    done_flops, n_blocks = 0.0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and (n_blocks + 1) * R <= S:
        r1 = S - n_blocks * R
        r0 = r1 - R
        oracle.partial_attention(q[:, r0:r1], k[:, :r1], v[:, :r1], r0, 0, True, row_block=R)
        # visible (query, key) pairs of rows r0..r1-1: sum of (pos + 1)
        done_flops += 4.0 * w.D * w.Hq * w.B * (R * r0 + R * (R + 1) / 2)
        n_blocks += 1
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cpus_visible": len(os.sched_getaffinity(0)), "cpu": cpu, "seconds": round(dt, 2),
            "sample": f"{n_blocks} blocks of {R} consecutive query rows (the last {n_blocks * R} rows) x {w.Hq} "
                      f"heads of {w.name}, each row at its full causal context: oracle.partial_attention in fp64 "
                      f"on torch CPU (GEMM-shaped row blocks), {done_flops:.3e} FLOP in {dt:.1f} s on {threads} "
                      f"threads"}


def machine_id(torch) -> dict:
    import socket
    props = torch.cuda.get_device_properties(0)
    uuid = str(getattr(props, "uuid", "")) or None
    return {"host": socket.gethostname(), "gpu_uuid": uuid, "device": props.name}


def timed_reps(torch, stream, fn, reps: int, warm_ms: float = 50.0):
    """Median ms of ``reps`` calls of fn, each bracketed by events on ``stream``, after a warm-up of at
    least two calls and ~warm_ms (the GPU sat idle while inputs were drawn on the host, and cold
    calls run below the steady rate)."""
    for _ in range(2):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    for _ in range(min(200, int(warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
        fn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sorted(e[0].elapsed_time(e[1]) for e in ev)[reps // 2]


def decode_bytes(wd) -> dict:
    """Algorithmic HBM bytes of the split-KV decode of workload wd: the kernel reads K, V and Q and
    writes every chunk's partial (O and LSE); the merge reads the partials and writes O and LSE."""
    kv = 2 * wd.B * wd.Skv * wd.Hkv * wd.D * 2
    qb = wd.B * wd.Hq * wd.D * 2
    part = wd.n_chunks * wd.B * wd.Hq * (wd.D + 1) * 4
    outb = wd.B * wd.Hq * (wd.D + 1) * 4
    return {"kernel": kv + qb + part, "merge": part + outb, "total": kv + qb + 2 * part + outb}


def gbs(nbytes: float, ms: float) -> dict:
    g = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(g, 1), "frac_hbm": round(g / PEAK_HBM_GBS, 4)}


def time_decode(torch, cp, si, dev, stream, reps: int) -> dict:
    """The split-KV decode of the decode workload (kernel + merge) and its allocation-free form."""
    wd = si.WORKLOADS[DECODE]
    log(f"[bench] drawing {wd.name} inputs")
    dq, dk, dv = [t.to(dev) for t in si.make_qkv(wd)]
    dws = torch.empty(cp.splitkv_decode_workspace_size(dq, dk, wd.n_chunks), dtype=torch.uint8, device=dev)
    dout = torch.empty(wd.q_shape(), dtype=torch.float32, device=dev)
    dlse = torch.empty(wd.q_shape()[:3], dtype=torch.float32, device=dev)
    ms_d = timed_reps(torch, stream, lambda: cp.splitkv_decode(dq, dk, dv, wd.n_chunks, out=dout, lse=dlse,
                                                               workspace=dws), reps, warm_ms=60.0)
    ms_dn = timed_reps(torch, stream, lambda: cp.splitkv_decode_noalloc(dq, dk, dv, wd.n_chunks, dout, dlse), reps)
    nb = decode_bytes(wd)["total"]
    log(f"[bench] decode {ms_d:.3f} ms, no-alloc {ms_dn:.3f} ms")
    return {"wd": wd, "tensors": (dq, dk, dv, dout, dlse), "ms": ms_d, "ms_noalloc": ms_dn,
            "result": {"workload": wd.name, **gbs(nb, ms_d), "algorithmic_bytes": nb, "peak_GB/s": PEAK_HBM_GBS,
                       "noalloc": gbs(nb, ms_dn)}}


def ring_merge_bytes(w) -> int:
    """Algorithmic HBM bytes of the ring merge of workload w (causal, every rank a chunk): each of the
    P(P+1)/2 visible pairs' partial rows (O and LSE, fp32) read once, each owner's rows written once."""
    P = w.n_chunks
    return (P * (P + 1) // 2 + P) * w.chunk * w.Hq * w.B * 4 * (w.D + 1)


def merge_profile_values() -> dict:
    """Entries of the committed ring-merge profile summary of the current kernel sources."""
    return _summary_values(MERGE_FILE, keep_text=("machine_host", "machine_gpu_uuid"))


def decode_profile_values() -> dict:
    """Entries of the committed decode profile summary of the current kernel sources."""
    return _summary_values(DECODE_FILE, keep_text=("machine_host", "machine_gpu_uuid"))


def tf(flops: float, ms: float) -> dict:
    t = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(t, 2), "pct_bf16_peak": round(100 * t / PEAK_BF16_TFLOPS, 2)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the timed Pass-KV ring steps (profiling runs: every partial-kernel launch is then a "
                         "headline ring step)")
    ap.add_argument("--no-1m", action="store_true", help="skip the 1M-token workload leg (~1 minute)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the split-KV decode workload, --steps timed calls (decode profiling runs)")
    ap.add_argument("--merge-only", action="store_true",
                    help="only the 128K ring's merge over its per-pair partials, --steps timed calls (profiling runs)")
    ap.add_argument("--summarize-merge", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="kernel trace and HBM traffic of the ring merge, beside a plain --merge-only line")
    ap.add_argument("--summarize-decode", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="kernel trace and HBM traffic of the decode kernel and its merge, beside a plain "
                         "--decode-only line of the same machine")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB fp32 copy kernel (counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [CLOCK_DIR [SQ_DIR [RDREQ_DIR]]]: HBM traffic (shader clock, "
                         "MFMA busy fraction, read bytes by request size) from rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="kernel-trace summary of the headline kernel beside a plain bench line of the same machine")
    args = ap.parse_args(argv)

    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3, 4, 5):
            ap.error("--summarize-pmc takes FETCH_DIR WRITE_DIR [CLOCK_DIR [SQ_DIR [RDREQ_DIR]]]")
        return summarize_pmc(*args.summarize_pmc)
    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace)
    if args.summarize_decode:
        return summarize_decode(*args.summarize_decode)
    if args.summarize_merge:
        return summarize_merge(*args.summarize_merge)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "the simulated CP ranks all run on one device.", file=sys.stderr)
        return 2

    import torch

    import context_attention_cpattn_amd as cp
    import seeded_inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    machine = machine_id(torch)
    if args.decode_only:
        # profiling runs of the decode workload alone: every decode kernel and merge launch is a C3 decode
        dec = time_decode(torch, cp, si, dev, torch.cuda.current_stream(dev), max(1, args.steps))
        line = {"decode": dec["result"], "machine": machine, "reps": max(1, args.steps)}
        if args.calibrate_copy:
            _copy_calibration(torch, dev)
            line["copy_calibration_bytes"] = COPY_BYTES
        print(json.dumps(line), flush=True)
        return 0
    w = si.WORKLOADS[PREFILL]
    log(f"[bench] {machine['device']} on {machine['host']}, {cp.version()}; drawing {w.name} inputs")
    q, k, v = si.make_qkv(w)
    gq, gk, gv = q.to(dev), k.to(dev), v.to(dev)
    P = w.n_chunks
    out = torch.empty(w.q_shape(), dtype=torch.float32, device=dev)
    lse = torch.empty(w.q_shape()[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)  # the stream the library launches on
    total_flops = w.flops()

    def ring_steps(order, ev=None):
        """One Pass-KV (or Pass-Q) ring: P accumulating ring-step launches, each pair merged into its
        owner's running (O, LSE) by the kernel that computes it."""
        for s in range(P):
            if ev is not None:
                ev[s][0].record(stream)
            cp.ring_step_accumulate(gq, gk, gv, P, s, out, lse, order, True)
            if ev is not None:
                ev[s][1].record(stream)

    if args.merge_only:
        # profiling runs of the ring merge alone: the 128K ring's per-pair partials once, then merges
        ws = torch.empty(cp.ring_prefill_workspace_size(gq, P, True), dtype=torch.uint8, device=dev)
        for s in range(P):
            cp.ring_step(gq, gk, gv, P, s, ws, "pass_kv", True)
        reps = max(1, args.steps)
        ms_m = timed_reps(torch, stream, lambda: cp.ring_merge(P, ws, out, lse, "pass_kv", True), reps)
        nb = ring_merge_bytes(w)
        line = {"ring_merge": {"workload": w.name, **gbs(nb, ms_m), "algorithmic_bytes": nb,
                               "peak_GB/s": PEAK_HBM_GBS}, "machine": machine, "reps": reps}
        log(f"[bench] ring merge {ms_m:.3f} ms")
        if args.calibrate_copy:
            _copy_calibration(torch, dev)
            line["copy_calibration_bytes"] = COPY_BYTES
        print(json.dumps(line), flush=True)
        return 0

    # ---- headline: the Pass-KV ring, one accumulating launch per ring step
    step_flops = ring_step_flops(w, "pass_kv")
    assert abs(sum(step_flops) - total_flops) / total_flops < 1e-9
    for _ in range(args.warmup):
        ring_steps("pass_kv")
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(P)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        ring_steps("pass_kv", events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = total_flops / (wall / args.steps) / 1e12
    k_ms = [[events[i][s][0].elapsed_time(events[i][s][1]) for s in range(P)] for i in range(args.steps)]
    kern_ms_total = sum(sum(x) for x in k_ms)
    avg_launch_ms = kern_ms_total / (args.steps * P)
    achieved = total_flops * args.steps / (kern_ms_total * 1e-3) / 1e12
    traffic, sclk, mfma_busy, _ = read_pmc_summary()
    trace = trace_values()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "partial_bf16_fast_kernel<128, false> (accumulating ring step)", "launches_per_step": P,
                "avg_launch_ms": round(avg_launch_ms, 4), "algorithmic_flop_per_launch": total_flops / P,
                "basis": "HIP events around every ring-step launch of the timed steps, on the stream the library "
                         "launches on; this run's machine",
                "machine": machine}
    if trace:
        # the committed kernel trace of the same kernel source and launch pattern, with the machine it ran on
        roofline.update({"frac_profiled": trace.get("frac_profiled"),
                         "avg_launch_ms_profiled": trace.get("partial_kernel_avg_ms"),
                         "profiled_machine": trace.get("machine_host"),
                         "profiled_source": "profiles/partial_bf16_prefill_s128k_p16_trace.txt"})
    if sclk:
        roofline.update({"sclk_ghz_profiled": sclk, "mfma_busy_fraction_profiled": mfma_busy,
                         "counters_source": "profiles/partial_bf16_prefill_s128k_p16_traffic.txt"})
    per_step_tflops = [round(step_flops[s] / (sum(k_ms[i][s] for i in range(args.steps)) / args.steps * 1e-3) / 1e12, 1)
                       for s in range(P)]
    log(f"[bench] step {ms_per_step:.2f} ms, {value:.1f} TFLOP/s; partial kernel {achieved:.1f} TFLOP/s per launch")
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "order": "pass_kv", "launch": "16 accumulating ring-step launches "
                   "(cpattn_ring_step_accumulate), the merge in each launch's epilogue", "B": w.B, "S": w.Sq,
                   "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "n_chunks": P, "causal": True, "seed": w.seed,
                   "inputs": "N(0,1) rounded to bf16", "flop_per_step": total_flops},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "per_ring_step_tflops": per_step_tflops,
    }
    if args.headline_only:
        if args.calibrate_copy:
            _copy_calibration(torch, dev)
            result["copy_calibration_bytes"] = COPY_BYTES
        print(json.dumps(result), flush=True)
        return 0

    # ---- Pass-Q: the same ring with Q moving, one accumulating launch per ring step
    ms_q = timed_reps(torch, stream, lambda: ring_steps("pass_q"), max(3, args.steps // 2))
    result["pass_q"] = {**tf(total_flops, ms_q), "launch": "16 accumulating ring-step launches, Pass-Q schedule"}
    log(f"[bench] pass_q {ms_q:.2f} ms")

    # ---- the ring with per-pair partials in a workspace, then one merge launch (all owners)
    ws = torch.empty(cp.ring_prefill_workspace_size(gq, P, True), dtype=torch.uint8, device=dev)
    ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def ring_workspace(timed=False):
        for s in range(P):
            cp.ring_step(gq, gk, gv, P, s, ws, "pass_kv", True)
        if timed:
            ev_m[0].record(stream)
        cp.ring_merge(P, ws, out, lse, "pass_kv", True)
        if timed:
            ev_m[1].record(stream)

    ms_w = timed_reps(torch, stream, ring_workspace, max(3, args.steps // 2))
    merge_ms = []
    for _ in range(3):
        ring_workspace(True)
        torch.cuda.synchronize()
        merge_ms.append(ev_m[0].elapsed_time(ev_m[1]))
    merge_ms = sorted(merge_ms)[1]
    merge_bytes = ring_merge_bytes(w)
    result["ring_workspace"] = {**tf(total_flops, ms_w), "launch": "16 ring_step launches into per-pair workspace "
                                "slots, then one ring_merge launch",
                                "merge": {"ms": round(merge_ms, 4), "GB/s": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1),
                                          "frac_hbm": round(merge_bytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                          "algorithmic_bytes": merge_bytes}}
    mprof = merge_profile_values()
    if mprof:
        # the committed kernel trace and counters of the same kernel sources (another run, named machine)
        result["ring_workspace"]["merge"]["profiled"] = {
            "avg_ms": mprof.get("ring_merge_kernel_avg_ms"), "GB/s": mprof.get("ring_merge_GB/s"),
            "frac_hbm": mprof.get("frac_hbm_profiled"), "hbm_bytes": mprof.get("ring_merge_kernel_hbm_bytes"),
            "machine_gpu_uuid": mprof.get("machine_gpu_uuid"), "source": "profiles/ring_merge_s128k_p16.txt"}
    log(f"[bench] ring with workspace {ms_w:.2f} ms (merge {merge_ms:.3f} ms)")

    # ---- the whole ring as one call: per-owner walk, partials into the workspace, merged at the walk's end
    ms_r = timed_reps(torch, stream, lambda: cp.ring_prefill(gq, gk, gv, P, "pass_kv", True, out=out, lse=lse,
                                                             workspace=ws), max(3, args.steps // 2))
    result["ring_prefill"] = {**tf(total_flops, ms_r), "launch": "ring_prefill: one launch, each owner's query "
                              "tiles walk their visible K/V chunks writing every pair's partial, then merge them "
                              "in arrival order"}
    del ws
    log(f"[bench] ring_prefill {ms_r:.2f} ms")

    # ---- fused: every owner walks its visible keys once, merge online, one launch
    ms_f = timed_reps(torch, stream, lambda: cp.ring_prefill_fused(gq, gk, gv, P, True, out=out, lse=lse),
                      max(3, args.steps // 2))
    result["fused"] = {**tf(total_flops, ms_f), "launch": "ring_prefill_fused: one launch, each owner's visible "
                       "keys in one pass, merge online"}
    log(f"[bench] fused {ms_f:.2f} ms")
    del gq, gk, gv, out, lse
    torch.cuda.empty_cache()

    # ---- 8K-token GQA workload: whole ring prefills and the fused prefill
    w8 = si.WORKLOADS["gqa16_bf16_s8k_p8"]
    log(f"[bench] drawing {w8.name} inputs")
    x = [t.to(dev) for t in si.make_qkv(w8)]
    o8 = torch.empty(w8.q_shape(), dtype=torch.float32, device=dev)
    l8 = torch.empty(w8.q_shape()[:3], dtype=torch.float32, device=dev)
    ws8 = torch.empty(cp.ring_prefill_workspace_size(x[0], w8.n_chunks, True), dtype=torch.uint8, device=dev)
    reps = max(10, args.steps)
    ms8 = timed_reps(torch, stream, lambda: cp.ring_prefill(*x, w8.n_chunks, "pass_kv", True, out=o8, lse=l8,
                                                               workspace=ws8), reps)
    ms8f = timed_reps(torch, stream, lambda: cp.ring_prefill_fused(*x, w8.n_chunks, True, out=o8, lse=l8), reps)
    result["gqa_8k"] = {"workload": w8.name, "order": "pass_kv", **tf(w8.flops(), ms8), "flop": w8.flops(),
                        "launch": "ring_prefill: one launch, each owner's query tiles walk their visible K/V "
                        "chunks writing every pair's partial, then merge them in arrival order",
                        "fused": tf(w8.flops(), ms8f)}
    log(f"[bench] 8K ring {ms8:.3f} ms, fused {ms8f:.3f} ms")
    del x, o8, l8, ws8

    # ---- 2048 new tokens against a 131072-token cached context: the order chosen by exchanged bytes
    Sq, Skv = 2048, 131072 + 2048
    qs = si.draw_tensor(811, si.TENSOR_Q, (1, Sq, 16, 128), torch.bfloat16).to(dev)
    ks = si.draw_tensor(811, si.TENSOR_K, (1, Skv, 1, 128), torch.bfloat16).to(dev)
    vs = si.draw_tensor(811, si.TENSOR_V, (1, Skv, 1, 128), torch.bfloat16).to(dev)
    order, b_kv, b_q = cp.ring_select_order(qs, ks, 16, True)
    f_s = 4.0 * 128 * 16 * sum(Skv - Sq + i + 1 for i in range(Sq))
    os_ = torch.empty(1, Sq, 16, 128, dtype=torch.float32, device=dev)
    ls_ = torch.empty(1, Sq, 16, dtype=torch.float32, device=dev)
    ms_s = timed_reps(torch, stream, lambda: cp.ring_prefill(qs, ks, vs, 16, "auto", True, out=os_, lse=ls_), reps)
    ms_sf = timed_reps(torch, stream, lambda: cp.ring_prefill_fused(qs, ks, vs, 16, True, out=os_, lse=ls_), reps)
    result["suffix_2048_on_128k"] = {"workload": "2048 new tokens x 16/1 heads, D=128, against 131072 cached "
                                     "tokens, 16 chunks, bf16, seed 811", "order_selected": order,
                                     "exchanged_bytes": {"pass_kv": b_kv, "pass_q": b_q}, "flop": f_s,
                                     **tf(f_s, ms_s), "fused": tf(f_s, ms_sf)}
    log(f"[bench] 2048 on 128K ({order}) {ms_s:.3f} ms, fused {ms_sf:.3f} ms")
    del qs, ks, vs, os_, ls_

    # ---- split-KV decode, its allocation-free form, decode over CP cache shards, and the cache write
    dreps = max(20, args.steps)
    dec = time_decode(torch, cp, si, dev, stream, dreps)
    wd = dec["wd"]
    dq, dk, dv, dout, dlse = dec["tensors"]
    result["decode"] = dec["result"]
    prof = decode_profile_values()
    if prof:
        # the committed kernel trace and counters of the same kernel sources (another run, named machine)
        result["decode"]["profiled"] = {k_: prof.get(k_) for k_ in (
            "decode_kernel_avg_ms", "merge_kernel_avg_ms", "kernel_and_merge_GB/s", "frac_hbm_profiled",
            "decode_kernel_hbm_bytes", "merge_kernel_hbm_bytes", "machine_gpu_uuid")}
        result["decode"]["profiled"]["source"] = "profiles/decode_stream_b128_kv32k_p8.txt"
    kv_bytes = 2 * wd.B * wd.Skv * wd.Hkv * wd.D * 2
    dec_bytes = decode_bytes(wd)["total"]
    # the same cache as the KV shards of 8 CP ranks, each with room for 64 more tokens
    C = wd.Skv // wd.n_chunks
    ks8 = [torch.empty(wd.B, C + 64, wd.Hkv, wd.D, dtype=torch.bfloat16, device=dev) for _ in range(wd.n_chunks)]
    vs8 = [torch.empty_like(t) for t in ks8]
    ms_w8 = timed_reps(torch, stream, lambda: cp.kv_cache_write(dk, dv, wd.n_chunks, ks8, vs8), dreps)
    lens = [C] * wd.n_chunks
    cws = torch.empty(cp.cp_decode_workspace_size(dq, ks8), dtype=torch.uint8, device=dev)
    ms_cd = timed_reps(torch, stream, lambda: cp.cp_decode(dq, ks8, vs8, lens, out=dout, lse=dlse, workspace=cws),
                       dreps)
    result["cache_write"] = {"what": f"{wd.name} K/V written into {wd.n_chunks} shards of {C + 64} rows",
                             **gbs(2 * kv_bytes, ms_w8), "algorithmic_bytes": 2 * kv_bytes}
    result["cp_decode"] = {"what": f"{wd.name} new tokens against the {wd.n_chunks} shards",
                           **gbs(dec_bytes, ms_cd), "algorithmic_bytes": dec_bytes}
    log(f"[bench] cache write {ms_w8:.3f} ms, decode over shards {ms_cd:.3f} ms")
    del dec, dq, dk, dv, dout, dlse, ks8, vs8, cws
    torch.cuda.empty_cache()

    # ---- the 1M-token workload (Pass-KV ring with per-pair partials and merge, and the fused walk)
    if not args.no_1m:
        w1 = si.WORKLOADS["prefill_bf16_s1m_p8"]
        log(f"[bench] drawing {w1.name} inputs")
        x = [t.to(dev) for t in si.make_qkv(w1)]
        o1 = torch.empty(w1.q_shape(), dtype=torch.float32, device=dev)
        l1 = torch.empty(w1.q_shape()[:3], dtype=torch.float32, device=dev)
        ws1 = torch.empty(cp.ring_prefill_workspace_size(x[0], w1.n_chunks, True), dtype=torch.uint8, device=dev)
        res1 = {}
        for name, fn in (("ring_prefill", lambda: cp.ring_prefill(*x, w1.n_chunks, "pass_kv", True, out=o1, lse=l1,
                                                                  workspace=ws1)),
                         ("fused", lambda: cp.ring_prefill_fused(*x, w1.n_chunks, True, out=o1, lse=l1))):
            fn()
            torch.cuda.synchronize()
            ts = []
            for i in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
                log(f"[bench] {w1.name} {name} rep {i + 1}/3: {ts[-1]:.1f} ms")
            res1[name] = tf(w1.flops(), sorted(ts)[1])
        result["prefill_1m"] = {"workload": w1.name, "order": "pass_kv", "flop": w1.flops(), **res1["ring_prefill"],
                                "launch": "ring_prefill: every visible (Q chunk, K/V chunk) pair's partial in one "
                                "launch (chunks this long go per pair), then the ring merge in arrival order",
                                "fused": res1["fused"]}
        del x, o1, l1, ws1
        torch.cuda.empty_cache()

    if args.calibrate_copy:
        _copy_calibration(torch, dev)
        result["copy_calibration_bytes"] = COPY_BYTES

    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on the host (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def _copy_calibration(torch, dev) -> None:
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _prefill_workload():
    import seeded_inputs as si
    return si.WORKLOADS[PREFILL]


def _pmc_rows(d: str):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter: str, name_part: str):
    vals = [float(r["Counter_Value"]) for r in rows
            if r.get("Counter_Name") == counter and name_part in r.get("Kernel_Name", "")]
    return sum(vals) / len(vals) if vals else None, len(vals)


def _clock_ghz(rows, name_part: str):
    """Shader clock during a kernel's dispatches: GRBM_GUI_ACTIVE counts busy clocks summed over the
    8 XCDs (a plain copy kernel reads 8 x ~2.4 GHz on this chip), divided by the dispatch time."""
    cyc = dur = 0.0
    for r in rows:
        if r.get("Counter_Name") == "GRBM_GUI_ACTIVE" and name_part in r.get("Kernel_Name", ""):
            cyc += float(r["Counter_Value"])
            dur += float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return cyc / dur / 8.0 if dur > 0 else None


def _read_bytes_by_size(rows, name_part: str):
    """Bytes read from EA per dispatch from the request-size counters (128/64/32-byte requests)."""
    n, _ = _per_dispatch(rows, "TCC_EA0_RDREQ_sum", name_part)
    r128, _ = _per_dispatch(rows, "TCC_EA0_RDREQ_128B_sum", name_part)
    r64, _ = _per_dispatch(rows, "TCC_EA0_RDREQ_64B_sum", name_part)
    r32, _ = _per_dispatch(rows, "TCC_EA0_RDREQ_32B_sum", name_part)
    if None in (n, r128, r64, r32):
        return None, None
    return 128.0 * r128 + 64.0 * r64 + 32.0 * r32, n - r128 - r64 - r32


def summarize_pmc(fetch_dir: str, write_dir: str, clock_dir: str | None = None, sq_dir: str | None = None,
                  rdreq_dir: str | None = None) -> int:
    """HBM bytes per partial-kernel launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the 1 GiB copy kernel; with a third run of
    GRBM_GUI_ACTIVE, also the shader clock the partial kernel ran at; with a fourth run of
    GRBM_GUI_ACTIVE and SQ counters, the MFMA busy fraction and the instruction mix."""
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    f_k, nf = _per_dispatch(fr, "FETCH_SIZE", "partial_bf16_fast_kernel")
    w_k, nw = _per_dispatch(wr, "WRITE_SIZE", "partial_bf16_fast_kernel")
    # the copy kernel is torch's x * 1.0 over 1 GiB (MulFunctor); the fill that creates its
    # source reads nothing and must not enter the calibration
    f_c, _ = _per_dispatch(fr, "FETCH_SIZE", "MulFunctor")
    w_c, _ = _per_dispatch(wr, "WRITE_SIZE", "MulFunctor")
    if None in (f_k, w_k, f_c, w_c):
        raise SystemExit("missing counters for the partial kernel or the copy kernel")
    f_scale = COPY_BYTES / (f_c * 1024.0)
    w_scale = COPY_BYTES / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * f_scale
    write_b = w_k * 1024.0 * w_scale
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("# HBM traffic of partial_bf16_fast_kernel<128, false> per launch on the 128K-token workload, Pass-KV\n")
        f.write("# accumulating ring steps, from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of:\n")
        f.write(f"#   {PROFILE_CMD} --steps 1 --warmup 0 --calibrate-copy\n")
        f.write("# (every partial launch of that run is one Pass-KV ring step)\n")
        f.write("# each counter scaled by its reading for a plain 1 GiB fp32 copy kernel\n")
        f.write(f"kernel_source_sha256_16: {kernel_hash()}\n")
        f.write(f"dispatches: {nf} (FETCH) {nw} (WRITE)\n")
        f.write(f"fetch_kib_per_dispatch_raw: {f_k:.1f}\n")
        f.write(f"write_kib_per_dispatch_raw: {w_k:.1f}\n")
        f.write(f"copy_fetch_scale: {f_scale:.4f}\n")
        f.write(f"copy_write_scale: {w_scale:.4f}\n")
        f.write(f"fetch_bytes_per_launch: {fetch_b:.0f}\n")
        f.write(f"write_bytes_per_launch: {write_b:.0f}\n")
        f.write(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}\n")
        d_f, nd = _per_dispatch(fr, "FETCH_SIZE", "decode_stream_kernel")
        d_w, _ = _per_dispatch(wr, "WRITE_SIZE", "decode_stream_kernel")
        if d_f is not None and d_w is not None:
            f.write(f"# split-KV decode kernel of the same runs ({nd} dispatches), same calibration\n")
            f.write(f"decode_fetch_bytes_per_launch: {d_f * 1024.0 * f_scale:.0f}\n")
            f.write(f"decode_write_bytes_per_launch: {d_w * 1024.0 * w_scale:.0f}\n")
        m_f, nm = _per_dispatch(fr, "FETCH_SIZE", "ring_merge_kernel")
        m_w, _ = _per_dispatch(wr, "WRITE_SIZE", "ring_merge_kernel")
        if m_f is not None and m_w is not None:
            f.write(f"# ring merge kernel of the same runs ({nm} dispatch(es), every owner of one Pass-KV step each), "
                    "same calibration\n")
            f.write(f"ring_merge_fetch_bytes_per_launch: {m_f * 1024.0 * f_scale:.0f}\n")
            f.write(f"ring_merge_write_bytes_per_launch: {m_w * 1024.0 * w_scale:.0f}\n")
        if rdreq_dir:
            rr = _pmc_rows(rdreq_dir)
            f.write("# cross-check from a run with TCC_EA0_RDREQ_{,128B_,64B_,32B_}sum: bytes read = 128/64/32 x\n"
                    "# the requests of each size (no calibration; 'other' = requests of none of those sizes)\n")
            for label, part in (("partial", "partial_bf16_fast_kernel"), ("decode", "decode_stream_kernel"),
                                ("ring_merge", "ring_merge_kernel"), ("copy", "MulFunctor")):
                rb, other = _read_bytes_by_size(rr, part)
                if rb is not None:
                    f.write(f"{label}_read_bytes_by_request_size: {rb:.0f} (other requests: {other:.0f})\n")
        if clock_dir:
            cr = _pmc_rows(clock_dir)
            ck, cc = _clock_ghz(cr, "partial_bf16_fast_kernel"), _clock_ghz(cr, "MulFunctor")
            f.write("# shader clock from a third run with --pmc GRBM_GUI_ACTIVE: busy clocks / 8 XCDs / dispatch time\n")
            f.write(f"sclk_ghz_partial_kernel: {ck:.3f}\n")
            f.write(f"sclk_ghz_copy_kernel: {cc:.3f}\n")
        if sq_dir:
            sr = _pmc_rows(sq_dir)
            k = "partial_bf16_fast_kernel"
            tot = {}
            for name in ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA",
                         "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"):
                tot[name], _ = _per_dispatch(sr, name, k)
            if None in tot.values():
                raise SystemExit("missing SQ counters for the partial kernel")
            simds = 4 * 256
            f.write("# fourth run: --pmc GRBM_GUI_ACTIVE and SQ counters, averages per partial-kernel dispatch\n")
            for name, val in tot.items():
                f.write(f"{name.lower()}: {val:.0f}\n")
            f.write("# MFMA busy cycles per SIMD over the busy cycles of one XCD (GRBM_GUI_ACTIVE / 8)\n")
            f.write(f"mfma_busy_fraction: {tot['SQ_VALU_MFMA_BUSY_CYCLES'] / (tot['GRBM_GUI_ACTIVE'] / 8.0 * simds):.3f}\n")
            f.write(f"valu_insts_per_mfma: {tot['SQ_INSTS_VALU'] / tot['SQ_INSTS_MFMA']:.2f}  (SQ_INSTS_VALU counts MFMAs too)\n")
            f.write(f"lds_insts_per_mfma: {tot['SQ_INSTS_LDS'] / tot['SQ_INSTS_MFMA']:.2f}\n")
            f.write(f"salu_insts_per_mfma: {tot['SQ_INSTS_SALU'] / tot['SQ_INSTS_MFMA']:.2f}\n")
            f.write(f"lds_bank_conflict_cycles_per_lds_active_cycle: "
                    f"{tot['SQ_LDS_BANK_CONFLICT'] / tot['SQ_LDS_IDX_ACTIVE']:.3f}\n")
    print(open(TRAFFIC_FILE).read())
    return 0


def _trace_stats(trace_dir: str) -> dict:
    stats = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                stats[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]) / 1e6)
    if not stats:
        raise SystemExit(f"no *kernel_stats.csv under {trace_dir}")
    return stats


def _kernel_profile(trace_dir: str, fetch_dir: str, write_dir: str, kernels) -> dict:
    """Trace calls and average ms, and HBM bytes per dispatch (FETCH_SIZE and WRITE_SIZE scaled by a
    1 GiB copy kernel's readings), of each kernel (label, name part, name part to avoid or None)."""
    stats = _trace_stats(trace_dir)
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    f_c, _ = _per_dispatch(fr, "FETCH_SIZE", "MulFunctor")
    w_c, _ = _per_dispatch(wr, "WRITE_SIZE", "MulFunctor")
    if None in (f_c, w_c):
        raise SystemExit("missing counters for the copy kernel (run with --calibrate-copy)")
    out = {"copy_fetch_scale": COPY_BYTES / (f_c * 1024.0), "copy_write_scale": COPY_BYTES / (w_c * 1024.0)}

    def match(name, part, avoid):
        return part in name and (avoid is None or avoid not in name)

    for label, part, avoid in kernels:
        hits = [v for n, v in stats.items() if match(n, part, avoid)]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {part!r} in the trace, found {len(hits)}")
        fv = [float(r["Counter_Value"]) for r in fr
              if r.get("Counter_Name") == "FETCH_SIZE" and match(r.get("Kernel_Name", ""), part, avoid)]
        wv = [float(r["Counter_Value"]) for r in wr
              if r.get("Counter_Name") == "WRITE_SIZE" and match(r.get("Kernel_Name", ""), part, avoid)]
        if not fv or not wv:
            raise SystemExit(f"missing FETCH_SIZE/WRITE_SIZE for {part}")
        fb = sum(fv) / len(fv) * 1024.0 * out["copy_fetch_scale"]
        wb = sum(wv) / len(wv) * 1024.0 * out["copy_write_scale"]
        out[label] = {"calls": hits[0][0], "avg_ms": hits[0][1], "counted": len(fv), "fetch": fb, "write": wb}
    return out


def _write_kernel_lines(f, prof: dict, labels) -> None:
    f.write("# kernel trace (rocprofv3 --kernel-trace --stats): calls, average ms\n")
    for label in labels:
        f.write(f"{label}_calls: {prof[label]['calls']}\n")
        f.write(f"{label}_avg_ms: {prof[label]['avg_ms']:.4f}\n")
    f.write("# HBM traffic per dispatch: FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB copy kernel's readings\n")
    f.write(f"copy_fetch_scale: {prof['copy_fetch_scale']:.4f}\n")
    f.write(f"copy_write_scale: {prof['copy_write_scale']:.4f}\n")
    for label in labels:
        k = prof[label]
        f.write(f"{label}_dispatches_counted: {k['counted']}\n")
        f.write(f"{label}_fetch_bytes: {k['fetch']:.0f}\n")
        f.write(f"{label}_write_bytes: {k['write']:.0f}\n")
        f.write(f"{label}_hbm_bytes: {k['fetch'] + k['write']:.0f}\n")


def _last_json(path: str) -> dict:
    return json.loads([ln for ln in open(path).read().splitlines() if ln.startswith("{")][-1])


def summarize_decode(trace_dir: str, fetch_dir: str, write_dir: str, bench_json: str) -> int:
    """Kernel trace and HBM traffic of the split-KV decode (decode_stream_kernel and the merge_kernel
    that follows it) from ``--decode-only`` runs under rocprofv3, beside the plain ``--decode-only``
    line of the same run."""
    import seeded_inputs as si
    wd = si.WORKLOADS[DECODE]
    nb = decode_bytes(wd)
    labels = ("decode_kernel", "merge_kernel")
    prof = _kernel_profile(trace_dir, fetch_dir, write_dir, (("decode_kernel", "decode_stream_kernel", None),
                                                             ("merge_kernel", "merge_kernel", "ring_merge")))
    b = _last_json(bench_json)
    kms, mms = prof["decode_kernel"]["avg_ms"], prof["merge_kernel"]["avg_ms"]
    g = nb["total"] / ((kms + mms) * 1e-3) / 1e9
    with open(DECODE_FILE, "w") as f:
        f.write(f"# Split-KV decode of {wd.name} (128 sequences x 1 new token, 16/1 heads, D = 128, 32768 cached\n")
        f.write("# tokens in 8 chunks): decode_stream_kernel, then merge_kernel over the 8 partials.\n")
        f.write("# On the MI355X machine, from /tmp with TMPDIR=/tmp, R = repository root, OUT = an output directory:\n")
        f.write(f"#   {DECODE_PROFILE_CMD} --steps 20 > $OUT/decode_plain.json\n")
        f.write(f"#   rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/dtrace -o kt -- {DECODE_PROFILE_CMD} --steps 20\n")
        f.write(f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/dfetch -o p -- {DECODE_PROFILE_CMD} --steps 3 --calibrate-copy\n")
        f.write(f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/dwrite -o p -- {DECODE_PROFILE_CMD} --steps 3 --calibrate-copy\n")
        f.write("#   python $R/bench.py --summarize-decode $OUT/dtrace $OUT/dfetch $OUT/dwrite $OUT/decode_plain.json\n")
        f.write(f"kernel_source_sha256_16: {kernel_hash()}\n")
        f.write(f"machine_host: {b['machine']['host']}\n")
        f.write(f"machine_gpu_uuid: {b['machine']['gpu_uuid']}\n")
        f.write("# algorithmic bytes: K + V + Q read and the partials written by the kernel; partials read and\n")
        f.write("# O + LSE written by the merge\n")
        f.write(f"decode_kernel_algorithmic_bytes: {nb['kernel']}\n")
        f.write(f"merge_kernel_algorithmic_bytes: {nb['merge']}\n")
        _write_kernel_lines(f, prof, labels)
        f.write("# rates from the trace averages against the algorithmic bytes\n")
        f.write(f"decode_kernel_GB/s: {nb['kernel'] / (kms * 1e-3) / 1e9:.1f}\n")
        f.write(f"kernel_and_merge_GB/s: {g:.1f}\n")
        f.write(f"frac_hbm_profiled: {g / PEAK_HBM_GBS:.4f}\n")
        f.write("# the plain --decode-only line of the same call (HIP events, median of the timed calls)\n")
        f.write(f"bench_decode_ms: {b['decode']['ms']}\n")
        f.write(f"bench_decode_GB/s: {b['decode']['GB/s']}\n")
        f.write(f"bench_decode_frac_hbm: {b['decode']['frac_hbm']}\n")
    print(open(DECODE_FILE).read())
    return 0


def summarize_merge(trace_dir: str, fetch_dir: str, write_dir: str, bench_json: str) -> int:
    """Kernel trace and HBM traffic of the ring merge of the 128K workload (ring_merge_kernel over the
    136 per-pair partials of a Pass-KV ring) from ``--merge-only`` runs under rocprofv3, beside the
    plain ``--merge-only`` line of the same run."""
    import seeded_inputs as si
    w = si.WORKLOADS[PREFILL]
    nb = ring_merge_bytes(w)
    prof = _kernel_profile(trace_dir, fetch_dir, write_dir, (("ring_merge_kernel", "ring_merge_kernel", None),))
    b = _last_json(bench_json)
    ms = prof["ring_merge_kernel"]["avg_ms"]
    g = nb / (ms * 1e-3) / 1e9
    with open(MERGE_FILE, "w") as f:
        f.write(f"# Ring merge of {w.name}: ring_merge_kernel merging each of the 16 owners' partials\n")
        f.write("# (136 per-pair slots of 8192 rows x 16 heads, fp32 O + LSE) in Pass-KV arrival order.\n")
        f.write("# On the MI355X machine, from /tmp with TMPDIR=/tmp, R = repository root, OUT = an output directory:\n")
        f.write(f"#   {MERGE_PROFILE_CMD} --steps 10 > $OUT/merge_plain.json\n")
        f.write(f"#   rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/mtrace -o kt -- {MERGE_PROFILE_CMD} --steps 10\n")
        f.write(f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/mfetch -o p -- {MERGE_PROFILE_CMD} --steps 3 --calibrate-copy\n")
        f.write(f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/mwrite -o p -- {MERGE_PROFILE_CMD} --steps 3 --calibrate-copy\n")
        f.write("#   python $R/bench.py --summarize-merge $OUT/mtrace $OUT/mfetch $OUT/mwrite $OUT/merge_plain.json\n")
        f.write(f"kernel_source_sha256_16: {kernel_hash()}\n")
        f.write(f"machine_host: {b['machine']['host']}\n")
        f.write(f"machine_gpu_uuid: {b['machine']['gpu_uuid']}\n")
        f.write("# algorithmic bytes: every slot's O and LSE read once, each owner's O and LSE written once\n")
        f.write(f"ring_merge_kernel_algorithmic_bytes: {nb}\n")
        _write_kernel_lines(f, prof, ("ring_merge_kernel",))
        f.write("# rate from the trace average against the algorithmic bytes\n")
        f.write(f"ring_merge_GB/s: {g:.1f}\n")
        f.write(f"frac_hbm_profiled: {g / PEAK_HBM_GBS:.4f}\n")
        f.write("# the plain --merge-only line of the same call (HIP events, median of the timed calls)\n")
        f.write(f"bench_merge_ms: {b['ring_merge']['ms']}\n")
        f.write(f"bench_merge_GB/s: {b['ring_merge']['GB/s']}\n")
        f.write(f"bench_merge_frac_hbm: {b['ring_merge']['frac_hbm']}\n")
    print(open(MERGE_FILE).read())
    return 0


def summarize_trace(trace_dir: str, bench_json: str) -> int:
    """Kernel-trace summary of the headline kernel (``rocprofv3 --kernel-trace --stats`` of the
    headline-only bench) next to the plain bench line taken in the same run on the same machine."""
    w = _prefill_workload()
    stats = {}
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                stats[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"]))
    part = [(n, v) for n, v in stats.items() if "partial_bf16_fast_kernel" in n]
    if not part:
        raise SystemExit(f"no partial_bf16_fast_kernel dispatches in {trace_dir}")
    calls = sum(v[0] for _, v in part)
    avg_ns = sum(v[2] for _, v in part) / calls
    line = json.loads([ln for ln in open(bench_json) if ln.strip().startswith("{")][-1])
    rl = line["roofline"]
    flop_launch = w.flops() / w.n_chunks
    tfl = flop_launch / (avg_ns * 1e-9) / 1e12
    os.makedirs(os.path.dirname(TRACE_FILE), exist_ok=True)
    with open(TRACE_FILE, "w") as f:
        f.write("# Kernel trace of the headline: 128K-token Pass-KV ring, 16 accumulating ring-step launches per step.\n")
        f.write("# On the MI355X machine, from /tmp with TMPDIR=/tmp, R = repository root, OUT = an output directory:\n")
        f.write(f"#   rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/trace -o kt -- "
                f"{PROFILE_CMD} --steps 5 --warmup 1\n")
        f.write(f"#   python $R/bench.py --summarize-trace $OUT/trace $OUT/bench_plain.json\n")
        f.write("# where $OUT/bench_plain.json is the plain `python $R/bench.py` line of the same call (same machine).\n")
        f.write(f"kernel_source_sha256_16: {kernel_hash()}\n")
        f.write(f"machine_host: {line['roofline'].get('machine', {}).get('host')}\n")
        f.write(f"machine_gpu_uuid: {line['roofline'].get('machine', {}).get('gpu_uuid')}\n")
        f.write(f"partial_kernel_dispatches: {calls}\n")
        f.write(f"partial_kernel_avg_ms: {avg_ns / 1e6:.4f}\n")
        f.write(f"flop_per_launch: {flop_launch:.6e}\n")
        f.write(f"tflops_profiled: {tfl:.1f}\n")
        f.write(f"frac_profiled: {tfl / PEAK_BF16_TFLOPS:.4f}\n")
        f.write(f"trace_kernel_ms_per_step: {avg_ns * w.n_chunks / 1e6:.3f}\n")
        f.write("# (the traced run has the profiler attached and runs after the plain bench; the clock the\n"
                "# chip holds moves between the runs, so its launches read a little longer or shorter)\n")
        f.write("# the plain bench line of the same call (HIP events around each launch; no profiler attached)\n")
        f.write(f"bench_ms_per_step: {line['ms_per_step']}\n")
        f.write(f"bench_value_tflops: {line['value']}\n")
        f.write(f"bench_avg_launch_ms: {rl['avg_launch_ms']}\n")
        f.write(f"bench_frac: {rl['frac']}\n")
        f.write("# every kernel of the traced run: calls, average ms\n")
        for n, (c, a_ns, _) in sorted(stats.items(), key=lambda kv_: -kv_[1][2]):
            short = n.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0][:90]
            f.write(f"kernel {short}: {c} {a_ns / 1e6:.4f}\n")
    print(open(TRACE_FILE).read())
    return 0


if __name__ == "__main__":
    sys.exit(main())
