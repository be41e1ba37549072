#!/usr/bin/env python3
"""Benchmark of the fused randomized Hadamard rotation + 4-bit quantisation on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only] [--given]

A step is one rhtq_forward call over one batch of the workload (rotation, scale,
quantisation and packing of every row; for NVFP4 also the tensor-amax pass).
Inputs are generated on the device before timing and rotate through enough
buffer sets (>= 512 MB) that the 256 MB Infinity Cache cannot hold them, so the
timed region reads HBM.  Timing uses HIP events on the stream the kernels run on.
The K timed steps are captured once into a HIP graph and the replay is timed
(--no-graph: eager launches), so that the host's per-call cost does not stretch
a kernel of a few microseconds; the eager time is reported beside it.

Prints ONE JSON line (rank 0).  `value` is tokens/s of the headline workload
(2048 x 4096 bf16, per-token INT4); the d=12288, KV, NVFP4 (dynamic and with a
given tensor scale), MXFP4, block-diagonal and d=11008 workloads and the KV
inverse are reported under "also", and a plain 512 MiB device copy under
"hbm_copy" as the bandwidth a streaming kernel reaches in practice.  For the 4096- and
12288-wide workloads, "same_grid_stream_floor" times rhtq_stream_floor: the same bytes moved
with the forward kernel's grid and access pattern and no arithmetic, the floor of that shape.  The CPU oracle, timed on a bounded sample on the host,
is reported as "cpu_baseline" (a baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RHT+4-bit quant tokens/s & HBM GB/s (% of peak) at d=4096 and d=12288"
HBM_PEAK_GBS = 8000.0
CACHE_DEFEAT_BYTES = 512 << 20
HEADLINE = "llama_4096_int4"
OTHERS = ["downproj_12288_int4g128", "kv_128_int4g128", "nvfp4_4096", "mxfp4_4096", "blockh128_4096_int4g128",
          "downproj7b_11008_int4g128", "wide172_22016_int4g128", "llama_4096_int4_f16", "llama_4096_int4_f32"]
KERNEL_SOURCES = ["randomized_hadamard_rotation_amd/csrc/rhtq_fast.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_fast12.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_fast24.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_fast2.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_fast172.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_fastw.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_epilogue.h",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_inverse_fast.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_device.h",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_generic.hip",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_internal.h",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_api.cpp",
                  "randomized_hadamard_rotation_amd/csrc/rhtq_floor.hip",
                  "include/rhtq.h",
                  "include/rhtq_floor.h",
                  "randomized_hadamard_rotation_amd/build.py"]   # compiler flags shape the kernels too


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def run_timed(torch, step, steps, warmup, graph):
    """Event-timed K steps on the current stream, after W untimed ones.  Returns (ms per step as
    reported, eager ms per step).  graph=True captures the K steps once into a HIP graph
    (torch.cuda.CUDAGraph) and times its replay: every step is still one full call on its own
    buffers, but the host's per-call cost (Python, ctypes) no longer stretches the measurement of
    a kernel that runs for a few microseconds.  The graph is replayed untimed for about 25 ms
    before the timed replay, so that the timed steps run at the GPU's steady clocks."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(run):
        stream = torch.cuda.current_stream()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        run()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    ms_eager = timed(lambda: [step(i) for i in range(steps)])
    if not graph:
        return ms_eager, ms_eager
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    # untimed replays for about 25 ms first: a timed region of a few dozen microseconds right
    # after start-up otherwise catches the GPU before its clocks have settled, and run-to-run
    # spread then exceeds the differences being measured
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > 0.025:
            break
    return timed(g.replay), ms_eager


def time_workload(R, torch, name, steps, warmup, graph=True, given=False, sha=False):
    """given=True (NVFP4 only): the tensor scale is the caller's (read, not computed), so one
    launch per step; it is set from one dynamic call on the same input before timing."""
    from workloads import WORKLOADS, bytes_per_call, generate
    w = WORKLOADS[name]
    assert not given or w.fmt == "nvfp4"
    x0, signs = generate(w, "cuda")
    input_sha = None
    if sha:
        from workloads import sha256_of
        input_sha = sha256_of(x0)
    nbytes = bytes_per_call(w, tensor_scale_dynamic=not given)
    sets = max(1, min(32, math.ceil(CACHE_DEFEAT_BYTES / nbytes)))
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    s_dev = torch.from_numpy(signs).to("cuda")
    outs = []
    for _ in range(sets):
        packed = torch.empty((w.tokens, w.n // 2), dtype=torch.uint8, device="cuda")
        sdt = {"f32": torch.float32, "f16": torch.float16, "e4m3": torch.uint8, "e8m0": torch.uint8}[w.scale_dtype]
        ng = 1 if w.group == 0 else w.n // w.group
        scales = torch.empty((w.tokens, ng), dtype=sdt, device="cuda")
        ts = torch.zeros(1, dtype=torch.float32, device="cuda") if w.fmt == "nvfp4" else None
        outs.append((packed, scales, ts))
    if given:
        g = R.rhtq_forward(x0, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)[2]
        for _, _, ts in outs:
            ts.copy_(g)
    mode = "given" if given else "dynamic"
    def step(i):   # on the current stream (the capture stream while a graph is recorded)
        packed, scales, ts = outs[i % sets]
        R.rhtq_forward(xs[i % sets], s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype,
                       tensor_scale=ts, tensor_scale_mode=mode, packed=packed, scales=scales,
                       block=w.block or None)

    ms, ms_eager = run_timed(torch, step, steps, warmup, graph)
    tokens = w.tokens * w.tokens_per_row
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": name + (" (given g)" if given else ""), "tokens": int(tokens), "rows": w.tokens, "n": w.n,
        "in_dtype": w.in_dtype, "fmt": w.fmt, "group": w.group, "scale_dtype": w.scale_dtype,
        "buffer_sets": sets, "ms_per_step": ms, "eager_ms_per_step": ms_eager,
        "launch": "hip-graph replay" if graph else "eager", "tokens_per_s": tokens / (ms * 1e-3),
        "rows_per_s": w.tokens / (ms * 1e-3), "bytes_per_call": nbytes, "achieved_gbs": gbs,
        "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
        "launches_per_step": 3 if w.fmt == "nvfp4" and not given else 1,
        **({"input_sha256": input_sha} if input_sha else {}),
    }


def time_floor(R, torch, name, steps, warmup, graph=True):
    """The streaming floor of the workload's launch shape (rhtq_stream_floor): the forward
    kernel's grid, workgroup shape and access pattern moving the same bytes, with no arithmetic
    beyond XOR folds.  Timed exactly as the workload is (same buffer-set rotation, graph replay)."""
    from workloads import WORKLOADS, bytes_per_call
    w = WORKLOADS[name]
    nbytes = bytes_per_call(w)
    sets = max(1, min(32, math.ceil(CACHE_DEFEAT_BYTES / nbytes)))
    gen = torch.Generator(device="cuda").manual_seed(1)
    xs = [torch.randn((w.tokens, w.n), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(sets)]
    ng = 1 if w.group == 0 else w.n // w.group
    sbytes = ng * {"f32": 4, "f16": 2}[w.scale_dtype]
    outs = [(torch.empty((w.tokens, w.n // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((w.tokens, sbytes // 4), dtype=torch.int32, device="cuda")) for _ in range(sets)]

    def step(i):
        packed, scales = outs[i % sets]
        R.rhtq_stream_floor(xs[i % sets], packed, scales)

    ms, ms_eager = run_timed(torch, step, steps, warmup, graph)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "rhtq_stream_floor: same grid, workgroup shape and 16-byte non-temporal loads as the "
                      "forward kernel, same bytes, XOR folds only", "ms_per_step": ms,
            "bytes_per_call": nbytes, "achieved_gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}


FLOORED = ["llama_4096_int4", "downproj_12288_int4g128"]   # widths rhtq_stream_floor covers
INVERSE = ["kv_128_int4g128"]
GIVEN = ["nvfp4_4096"]   # NVFP4 with the caller's tensor scale: one pass over x


def time_inverse(R, torch, name, steps, warmup, graph=True):
    """The KV-cache read path: rhtq_inverse of the workload's own codes (fp32 output)."""
    from workloads import WORKLOADS, generate
    w = WORKLOADS[name]
    x0, signs = generate(w, "cuda")
    s_dev = torch.from_numpy(signs).to("cuda")
    packed, scales, ts = R.rhtq_forward(x0, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
    del x0
    nbytes = packed.numel() + scales.numel() * scales.element_size() + w.tokens * w.n * 4
    sets = max(1, min(8, math.ceil(CACHE_DEFEAT_BYTES / nbytes)))
    outs = [torch.empty((w.tokens, w.n), dtype=torch.float32, device="cuda") for _ in range(sets)]
    def step(i):
        R.rhtq_inverse(packed, scales, w.n, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype,
                       tensor_scale=ts, out=outs[i % sets])

    ms, ms_eager = run_timed(torch, step, steps, warmup, graph)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": name + " (inverse)", "rows": w.tokens, "n": w.n, "fmt": w.fmt, "group": w.group,
            "ms_per_step": ms, "eager_ms_per_step": ms_eager, "launch": "hip-graph replay" if graph else "eager",
            "rows_per_s": w.tokens / (ms * 1e-3), "bytes_per_call": nbytes,
            "achieved_gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}


def _oracle_reps(args):
    """One process's share of the CPU baseline: the workload's full input (drawn here from the
    same seeds) through the oracle, untouched, repeated until the budget is spent.
    Returns (repetitions, seconds)."""
    name, budget_s = args
    import numpy as np
    import oracle as O
    from workloads import WORKLOADS, generate
    w = WORKLOADS[name]
    x, s = generate(w, "cpu")
    xr = x.float().numpy().astype(np.float64)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.forward(xr, s, w.fmt, w.group, w.scale_dtype)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def cpu_baseline(name, budget_s=10.0, procs=None):
    """The oracle, untouched, on the host: `procs` fresh single-threaded interpreters (one per
    core this process may use, at most 16), each running the full workload input through the
    oracle for the same budget at the same time; `value` is the sum of their rates.  The same
    in this one process is reported beside it.  Runs before anything touches the GPU."""
    import multiprocessing
    from workloads import WORKLOADS
    w = WORKLOADS[name]
    per_input = w.tokens * w.tokens_per_row
    reps, el = _oracle_reps((name, budget_s))
    one = reps * per_input / el
    procs = procs or max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                                else os.cpu_count() or 1))
    env_before = os.environ.get("OMP_NUM_THREADS")
    os.environ["OMP_NUM_THREADS"] = "1"   # read by the children at their NumPy import
    try:
        with multiprocessing.get_context("spawn").Pool(procs) as pool:
            res = pool.map(_oracle_reps, [(name, budget_s)] * procs)
    finally:
        if env_before is None:
            os.environ.pop("OMP_NUM_THREADS", None)
        else:
            os.environ["OMP_NUM_THREADS"] = env_before
    pooled = sum(r * per_input / e for r, e in res)
    return {"value": pooled, "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "cores_note": "the pool is capped at 16 processes: the GPU host's share of CPU per GPU is 16 "
                          "cores, whatever os.cpu_count() reports for the whole machine",
            "sample": f"{procs} single-threaded processes at once, each repeating the numpy fp64 oracle over the "
                      f"full {w.tokens}x{w.n} {w.in_dtype} input of {name} for {budget_s:.0f} s "
                      f"({sum(r for r, _ in res)} repetitions in all)",
            "single_process": {"value": one, "unit": "tokens/s", "cores": 1,
                               "sample": f"{reps} x the full input in this process ({el:.1f} s)"}}


def copy_bandwidth(torch, nbytes=512 << 20, reps=20):
    """A plain device-to-device copy (torch's copy kernel) of nbytes, event-timed: read plus
    write bytes per second, the bandwidth a streaming kernel can reach in practice on this GPU."""
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    return {"bytes": 2 * nbytes, "ms": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": 2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def copy_calibration(torch, nbytes=1 << 30, reps=8):
    """A plain device copy of known size (torch's elementwise negation of fp32, which reads
    and writes nbytes each): the HBM counters read under it give the factor that turns
    FETCH_SIZE / WRITE_SIZE into bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": nbytes, "write_bytes": nbytes, "reps": reps}}),
          flush=True)


def rocprof_summary(root, pattern):
    """Compact text summary of rocprofv3 CSV output under root: per kernel whose name
    contains pattern, the mean of each counter per dispatch and the kernel-trace stats."""
    import collections
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        acc = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if pattern in r.get("Kernel_Name", ""):
                    acc[r["Kernel_Name"]][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for k, cs in acc.items():
            for c, per in cs.items():
                xs = list(per.values())
                print(f"PMC {c} mean_per_dispatch {sum(xs) / len(xs):.6g} dispatches {len(xs)} kernel {k}")
    for f in sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)):
        durs = collections.defaultdict(list)
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if pattern in r["Kernel_Name"]:
                    durs[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        for k, ds in durs.items():
            ds.sort()
            q = lambda p: ds[min(len(ds) - 1, int(p * (len(ds) - 1) + 0.5))]
            print(f"TRACE calls {len(ds)} p10_ns {q(0.1)} median_ns {q(0.5)} p90_ns {q(0.9)} kernel {k}")
    for f in sorted(glob.glob(os.path.join(root, "**", "*kernel_stats.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if pattern in r["Name"]:
                    print(f"STATS calls {r['Calls']} avg_ns {float(r['AverageNs']):.1f} min_ns {r['MinNs']} "
                          f"max_ns {r['MaxNs']} total_ns {r.get('TotalDurationNs', '?')} kernel {r['Name']}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="time only --workload")
    ap.add_argument("--given", action="store_true", help="NVFP4 workload with a given tensor scale")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="summarise rocprofv3 CSV output under DIR and exit (no GPU use)")
    ap.add_argument("--kernel-pattern", default="",
                    help="with --rocprof-summary: only kernels whose name contains this")
    args = ap.parse_args()

    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary, args.kernel_pattern)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: rows are independent, so the path shards "
              "by rows with no exchange, and this benchmark measures one GPU's share.",
              file=sys.stderr)
        sys.exit(2)

    # the oracle's CPU baseline first, while no process has touched the GPU
    cpu = None if (args.no_cpu_baseline or args.copy_calibration) else cpu_baseline(args.workload)

    import torch
    import randomized_hadamard_rotation_amd as R
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return

    graph = not args.no_graph
    head = time_workload(R, torch, args.workload, args.steps, args.warmup, graph, given=args.given, sha=True)
    if args.workload in FLOORED and not args.given:
        head["same_grid_stream_floor"] = time_floor(R, torch, args.workload, args.steps, args.warmup, graph)
    also = []
    if not args.only:
        for name in OTHERS:
            if name != args.workload:
                rec = time_workload(R, torch, name, args.steps, args.warmup, graph)
                if name in FLOORED:
                    rec["same_grid_stream_floor"] = time_floor(R, torch, name, args.steps, args.warmup, graph)
                    rec["over_floor"] = rec["ms_per_step"] / rec["same_grid_stream_floor"]["ms_per_step"]
                also.append(rec)
        for name in GIVEN:
            also.append(time_workload(R, torch, name, args.steps, args.warmup, graph, given=True))
        for name in INVERSE:
            also.append(time_inverse(R, torch, name, args.steps, args.warmup, graph))

    per_launch_ms = head["ms_per_step"] / head["launches_per_step"]
    traffic = traffic_for(args.workload + ("_given" if args.given else ""))
    roofline = {"bound": "hbm", "achieved": head["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": head["achieved_gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                "kernel_ms": per_launch_ms, "algorithmic_bytes_per_launch": head["bytes_per_call"]}
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": "bf16 input; fp32 accumulation; the second matrix-core stage carries each value as two f16 "
                      "terms under a power-of-two scale (22 significant bits); the worst rotation error against "
                      "the fp64 oracle over every row of each workload is printed by tests/test_gpu_fullsize.py",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": head["tokens"], "n": head["n"],
                   "in_dtype": head["in_dtype"], "fmt": head["fmt"], "group": head["group"],
                   "scale_dtype": head["scale_dtype"], "buffer_sets": head["buffer_sets"],
                   "input_sha256": head["input_sha256"]},
        "hbm_gbs": head["achieved_gbs"],
        "launch": head["launch"],
        "eager_ms_per_step": head["eager_ms_per_step"],
        "roofline": roofline,
        **({"same_grid_stream_floor": {**head["same_grid_stream_floor"],
                                       "over_floor": head["ms_per_step"] / head["same_grid_stream_floor"]["ms_per_step"]}}
           if "same_grid_stream_floor" in head else {}),
        "also": also,
    }
    if not args.only:
        out["hbm_copy"] = copy_bandwidth(torch)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
