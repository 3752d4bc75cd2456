"""Benchmark of the block-scaled FP8 W8A16 GEMM on one MI355X.

One step = one GEMM call (the whole path: plan, weight stream, dequant,
MFMA, scale fold, split-K fix-up, BF16 store) on one batch of synthetic
input already resident in HBM.  The headline workload is M=8, N=4096,
K=4096 (FP8 weight, BF16 activations); the other workloads are reported
alongside in ``all_workloads``.

Weights are measured cold: every call reads a different replica of the
operands from an arena of >= 512 MiB (twice the 256 MiB Infinity Cache), so
the weight bytes come from HBM.  Time is taken with HIP events on the stream
the kernels run on, bracketed by device synchronisation.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only-main]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + µs/call, W8A16 GEMM at M=1..32"
MAIN_WORKLOAD = "m8_n4096_k4096"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense BF16 MFMA
ARENA_BYTES = 512 << 20
NOTE = ("The source pages give tile and shared-memory constants for GB10 (sm_121) "
        "and Hopper kernels but no throughput figures, so there is no published "
        "number to compare against.")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp8_w8a16_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def log(msg: str):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Arena:
    """R replicas of one problem's operands on the GPU."""

    def __init__(self, torch, prob, replicas: int):
        dev = torch.device("cuda")
        self.prob = prob
        self.r = replicas
        a = torch.from_numpy(prob.a).view(torch.int16).to(dev)
        w = torch.from_numpy(prob.w).to(dev)
        s = torch.from_numpy(prob.scale).to(dev)
        c = torch.from_numpy(prob.c).view(torch.int16).to(dev)
        self.a = a.reshape(1, -1).repeat(replicas, 1)
        self.w = w.reshape(1, -1).repeat(replicas, 1)
        self.s = s.reshape(1, -1).repeat(replicas, 1)
        self.c = c.reshape(1, -1).repeat(replicas, 1)
        self.ptrs = [(self.a[i].data_ptr(), self.w[i].data_ptr(), self.s[i].data_ptr(),
                      self.c[i].data_ptr()) for i in range(replicas)]


def time_workload(torch, w8, prob, steps: int, warmup: int, cold: bool = True,
                  plan=None):
    per_replica = (prob.a.nbytes + prob.w.nbytes + prob.scale.nbytes + prob.c.nbytes)
    replicas = max(1, -(-ARENA_BYTES // per_replica)) if cold else 1
    arena = Arena(torch, prob, replicas)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    lib_args = (prob.a_row_stride, prob.c_row_stride, prob.m, prob.n, prob.k)

    def call(i):
        a, w, s, c = arena.ptrs[i % replicas]
        st = w8.gemm_raw(a, lib_args[0], w, s, c, lib_args[1], lib_args[2], lib_args[3],
                         lib_args[4], sp, plan)
        if st != 0:
            raise RuntimeError("w8a16_gemm failed: %d %s" % (st, w8.last_error()))

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        call(warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop)
    return arena, ms / steps, wall, replicas


def check_arena_output(arena, oracle, datagen, torch):
    """Sampled parity of the last replica written by the timed loop."""
    p = arena.prob
    import numpy as np
    c = arena.c[0].cpu().numpy().view(np.uint16).reshape(p.c.shape)
    rows, cols = datagen.sample_indices(p.m, p.n, 512, seed=99)
    oc, _, bound = oracle.gemm_at(p.a, p.w, p.scale, p.m, p.n, p.k, rows, cols,
                                  a_row_stride=p.a_row_stride)
    ok = oracle.within_tolerance(c[rows, cols], oc, bound)
    return bool(ok.all())


def cpu_baseline(oracle, datagen, prob, budget_s: float = 10.0):
    """The oracle as it stands, on the host cores, over whole GEMMs of the
    headline workload, repeated until about `budget_s` seconds."""
    threads = len(os.sched_getaffinity(0))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm(prob.a, prob.w, prob.scale, prob.m, prob.n, prob.k,
                    a_row_stride=prob.a_row_stride, threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / reps
    return dt, reps, threads


def load_traffic(workload: str, kernel_hash: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_hash") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=MAIN_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-main", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--warm", action="store_true",
                    help="reuse one set of buffers (weights may stay in cache)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this GEMM runs on one GPU; multi-GPU runs (--gpus %d, "
              "WORLD_SIZE=%d) are not supported -- the operation shards along N "
              "with no exchange, so per-GPU throughput is the one-GPU figure."
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    import oracle

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w8.library()
    khash = kernel_source_hash()

    wl = datagen.workload(args.workload)
    log("generating %s" % wl.name)
    prob = datagen.make_workload(wl)
    plan = w8.plan(wl.m, wl.n, wl.k, torch.cuda.get_device_properties(0).multi_processor_count)
    log("timing %s plan=%s" % (wl.name, plan.as_dict()))
    arena, ms_call, wall, replicas = time_workload(torch, w8, prob, args.steps, args.warmup,
                                                   cold=not args.warm)
    parity_ok = check_arena_output(arena, oracle, datagen, torch)
    del arena
    torch.cuda.empty_cache()
    alg_bytes = wl.algorithmic_bytes()
    gbs = alg_bytes / (ms_call * 1e-3) / 1e9
    log("%s: %.3f us/call, %.1f GB/s (parity %s)" % (wl.name, ms_call * 1e3, gbs, parity_ok))

    traffic = load_traffic(wl.name, khash)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_call,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "m": wl.m, "n": wl.n, "k": wl.k,
                   "a_row_stride": wl.a_row_stride, "c_row_stride": wl.c_row_stride,
                   "seed": wl.seed, "weights": "warm" if args.warm else "cold",
                   "arena_replicas": replicas},
        "us_per_call": round(ms_call * 1e3, 3),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tflops": round(wl.flops() / (ms_call * 1e-3) / 1e12, 3),
        "plan": plan.as_dict(),
        "parity_sampled_ok": parity_ok,
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "w8a16_stream_kernel" if plan.kernel == w8.KERNEL_STREAM
                      else "w8a16_tile_kernel",
            "algorithmic_bytes_per_launch": alg_bytes,
        },
        "kernel_source_hash": khash,
        "note": NOTE,
    }

    if not args.only_main:
        rows = []
        for other in datagen.WORKLOADS:
            if other.name == wl.name:
                rows.append({"workload": wl.name, "us_per_call": round(ms_call * 1e3, 3),
                             "gbs": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 2),
                             "tflops": result["tflops"],
                             "pct_mfma": round(100 * result["tflops"] / BF16_PEAK_TFLOPS, 2),
                             "parity_sampled_ok": parity_ok, "plan": plan.as_dict()})
                continue
            log("generating %s" % other.name)
            op = datagen.make_workload(other)
            oplan = w8.plan(other.m, other.n, other.k)
            steps = max(20, min(args.steps, 200))
            ar, oms, _, orep = time_workload(torch, w8, op, steps, max(5, args.warmup // 2))
            ok = check_arena_output(ar, oracle, datagen, torch)
            del ar
            torch.cuda.empty_cache()
            ogbs = other.algorithmic_bytes() / (oms * 1e-3) / 1e9
            otf = other.flops() / (oms * 1e-3) / 1e12
            log("%s: %.3f us/call, %.1f GB/s, %.1f TFLOP/s (parity %s)" %
                (other.name, oms * 1e3, ogbs, otf, ok))
            rows.append({"workload": other.name, "us_per_call": round(oms * 1e3, 3),
                         "gbs": round(ogbs, 1), "pct_hbm": round(100 * ogbs / HBM_PEAK_GBS, 2),
                         "tflops": round(otf, 3),
                         "pct_mfma": round(100 * otf / BF16_PEAK_TFLOPS, 2),
                         "parity_sampled_ok": ok, "plan": oplan.as_dict(),
                         "arena_replicas": orep})
            del op
        result["all_workloads"] = rows

    if not args.no_cpu:
        log("timing the CPU oracle on %s" % wl.name)
        dt, reps, threads = cpu_baseline(oracle, datagen, prob)
        result["cpu_baseline"] = {
            "value": round(alg_bytes / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "%d whole %s GEMMs (FP64 C oracle, OpenMP), %.3f s each" %
                      (reps, wl.name, dt),
            "us_per_call": round(dt * 1e6, 1),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
