"""Benchmark of the block-scaled FP8 W8A16 GEMM on one MI355X.

One step = one GEMM call (the whole path: plan, weight stream, dequant,
MFMA, scale fold, K-split reduction, BF16 store) on one batch of synthetic
input already resident in HBM.  The headline workload is M=8, N=4096,
K=4096 (FP8 weight, BF16 activations); the other workloads are reported
alongside in ``all_workloads``.

Weights are measured cold: every call reads a different replica of the
operands from an arena of >= 512 MiB (twice the 256 MiB Infinity Cache), so
the weight bytes come from HBM.  The K timed calls are captured once into a
HIP graph and replayed, so the host's per-call launch cost (about 3 us from
Python) cannot starve the GPU between kernels; time is taken with HIP events
on the stream the kernels run on, bracketed by device synchronisation.  The
same calls issued one by one (eager) are timed too and reported beside it.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only-main]
    python bench.py --traffic-run          (workload for rocprofv3 --pmc runs)
    python bench.py --m-sweep N K          (default plan for m = 1..256, one line each)
    python bench.py --batched              (Q/K/V arms in one batched call vs three calls)
    python bench.py --w8a8                 (FP8 activation quantizer + W8A8 GEMM)
    python bench.py --w4a4                 (W4A4 MX GEMV, tiled and persistent)
    python bench.py --trace-run WORKLOAD [K]   (the timed region alone, for rocprofv3)
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR WORKLOAD   (writes profiles/)
    python bench.py --summarize-trace TRACE_DIR WORKLOAD [K]          (writes profiles/)
    python bench.py --summarize-mfma PMC_DIR WORKLOAD                 (writes profiles/)
    python bench.py --summarize-pipeline ROOT                         (writes profiles/)
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
METRIC_W8A8 = "achieved HBM GB/s (% of peak) + µs/call, W8A8 GEMM (FP8 activations) at M=8..32"
METRIC_W4A4 = "achieved HBM GB/s (% of peak) + µs/call, W4A4 MXFP4 GEMV at M=8..32"
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


SCRUB_BYTES = 512 << 20       # twice the 256 MiB Infinity Cache
SPIN_UP_S = 0.02              # untimed GPU work right before a timed region


class Scrub:
    """A 512 MiB device buffer whose fill, enqueued right before a timed
    region, evicts the Infinity Cache: the replicas the timed calls read
    first then come from HBM, whatever the number of timed calls."""

    def __init__(self, torch):
        self.buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda")

    def run(self):
        self.buf.fill_(0x5A5A5A5A)


def time_workload(torch, w8, prob, steps: int, warmup: int, cold: bool = True,
                  plan=None, scrub=None):
    """Times `steps` calls: eagerly, then as one HIP graph of the same calls.
    Call i reads replica i mod R of the operands, R replicas spanning
    >= 512 MiB (twice the Infinity Cache).  Before each timed region the
    GPU runs about 20 ms of untimed calls (so it is at its working clock,
    not ramping up from idle) and then the 512 MiB scrub fill (so the first
    replicas are not cache-resident).  Returns (arena, graph ms per call,
    eager ms per call, replicas)."""
    per_replica = (prob.a.nbytes + prob.w.nbytes + prob.scale.nbytes + prob.c.nbytes)
    replicas = max(1, -(-ARENA_BYTES // per_replica)) if cold else 1
    arena = Arena(torch, prob, replicas)
    if cold and scrub is None:
        scrub = Scrub(torch)
    stream = torch.cuda.Stream()
    lib_args = (prob.a_row_stride, prob.c_row_stride, prob.m, prob.n, prob.k)

    def call(i):
        a, w, s, c = arena.ptrs[i % replicas]
        st = w8.gemm_raw(a, lib_args[0], w, s, c, lib_args[1], lib_args[2], lib_args[3],
                         lib_args[4], stream.cuda_stream, plan)
        if st != 0:
            raise RuntimeError("w8a16_gemm failed: %d %s" % (st, w8.last_error()))

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(warmup):          # also allocates any K-split workspace
            call(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                call(i)

        def spin_up():
            t0 = time.perf_counter()
            while True:
                graph.replay()
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= SPIN_UP_S:
                    break
            if scrub is not None:
                scrub.run()

        spin_up()
        start.record(stream)
        for i in range(steps):
            call(i)
        stop.record(stream)
        torch.cuda.synchronize()
        eager_ms = start.elapsed_time(stop) / steps
        spin_up()
        start.record(stream)
        graph.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(stop) / steps
    return arena, graph_ms, eager_ms, replicas


def trace_run(wl_name: str, steps: int = 20, warmup: int = 5):
    """The benchmark's timed region alone, for rocprofv3 --kernel-trace:
    warm-up calls, the spin-up graph replays and the timed graph replay of
    `steps` calls (each call on its own replica after the scrub), nothing
    else.  The summary keeps each kernel's last `steps` dispatches: the
    timed replay."""
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    w8.library()
    wl = datagen.workload(wl_name)
    prob = datagen.make_workload(wl)
    arena, ms, _, _ = time_workload(torch, w8, prob, steps, warmup)
    del arena
    print("trace run done: %s %.3f us/call (graph replay)" % (wl_name, ms * 1e3), flush=True)


def check_arena_output(arena, calls: int):
    """Sanity of every replica written by the `calls` timed and warm-up
    calls (call i writes replica i mod replicas): all m x n outputs
    finite BF16 and the pitch pad / extra rows still hold their sentinel.
    (Numerical parity against the oracle is the GPU tests' job; the timed
    legs of the benchmark do not run the oracle.)"""
    import numpy as np
    p = arena.prob
    ok = True
    for i in range(min(arena.r, calls)):
        c = arena.c[i].cpu().numpy().view(np.uint16).reshape(p.c.shape)
        body = c[:p.m, :p.n]
        ok &= bool(((body & 0x7F80) != 0x7F80).all())        # no Inf / NaN
        ok &= bool((c[:p.m, p.n:] == p.c[:p.m, p.n:]).all())
        ok &= bool((c[p.m:, :] == p.c[p.m:, :]).all())
    return ok


def cpu_baseline(oracle, datagen, prob, budget_s: float = 10.0, threads: int = 0):
    """The oracle as it stands, on the host cores (all of them unless
    `threads` is given), over whole GEMMs of the headline workload, repeated
    until about `budget_s` seconds."""
    threads = threads or len(os.sched_getaffinity(0))
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


def oracle_check(oracle, prob, c_bits, threads: int) -> dict:
    """The GPU's C (BF16 bits, whole buffer) against the whole oracle:
    fraction of outputs equal to the oracle's bits, the largest
    |gpu - exact| / B (B = sum |a*w*s| of the output; the BF16 rounding of
    the result is part of it), the largest error as a fraction of the
    parity bar 2^-8 * B + ulp(oracle), and whether every output passes."""
    import numpy as np
    m, n = prob.m, prob.n
    oc, tot, bound = oracle.gemm(prob.a, prob.w, prob.scale, m, n, prob.k,
                                 a_row_stride=prob.a_row_stride, threads=threads)
    g = c_bits[:m, :n]
    gv = oracle.bf16_bits_to_f64(g)
    ov = oracle.bf16_bits_to_f64(oc)
    pos = bound > 0
    err_b = float(np.max(np.abs(gv - tot)[pos] / bound[pos])) if pos.any() else 0.0
    bar = np.ldexp(bound, -8) + oracle.bf16_ulp(ov)
    return {"outputs": int(m * n), "bitexact_frac": round(float(np.mean(g == oc)), 6),
            "max_err_over_B": err_b,
            "max_err_over_bar": float(np.max(np.abs(gv - ov) / bar)),
            "within_tolerance": bool(oracle.within_tolerance(g, oc, bound).all())}


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


COPY_BYTES = 256 << 20


def traffic_run(wl_name: str):
    """A short run for rocprofv3 --pmc: the 512 MiB cache scrub, 20 cold calls
    of the workload (each on its own replica), then three plain device
    copies of COPY_BYTES (the counters' calibration)."""
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    wl = datagen.workload(wl_name)
    prob = datagen.make_workload(wl)
    per = prob.a.nbytes + prob.w.nbytes + prob.scale.nbytes + prob.c.nbytes
    replicas = max(1, -(-ARENA_BYTES // per))
    arena = Arena(torch, prob, replicas)
    Scrub(torch).run()             # the first replicas are not cache-resident
    sp = torch.cuda.current_stream().cuda_stream
    for i in range(20):
        a, w, s, c = arena.ptrs[i % replicas]
        st = w8.gemm_raw(a, prob.a_row_stride, w, s, c, prob.c_row_stride, prob.m, prob.n,
                         prob.k, sp)
        if st != 0:
            raise RuntimeError(w8.last_error())
    torch.cuda.synchronize()
    del arena
    torch.cuda.empty_cache()
    src = torch.ones(COPY_BYTES // 8, dtype=torch.float64, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("traffic run done", flush=True)


def _pmc_values(directory: str, counter: str):
    """Per-dispatch counter values by kernel name, from a rocprofv3 CSV."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


PIPELINE_GROUPS = (
    "TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum "
    "TCP_UTCL1_TRANSLATION_MISS_sum",
    "TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum TD_TD_BUSY_sum TD_TC_STALL_sum",
    "TCP_UTCL1_TRANSLATION_HIT_sum TCP_UTCL1_STALL_MULTI_MISS_sum TCP_TCR_TCP_STALL_CYCLES_sum "
    "TCP_TCP_TA_DATA_STALL_CYCLES_sum",
    "TCC_HIT_sum TCC_MISS_sum TCC_TAG_STALL_sum GRBM_GUI_ACTIVE",
)
PIPELINE_WORKLOADS = ("m8_n4096_k4096", "m16_n12288_k5120", "m32_n6144_k2048_strided",
                      "m128_n8192_k8192")


def summarize_pipeline(root: str):
    """Writes profiles/memory_pipeline_counters.txt from the rocprofv3 PMC
    runs ROOT/<workload>_g<i> (counter group i of PIPELINE_GROUPS, each a
    --traffic-run of the workload): per GEMM kernel, each counter's mean over
    its dispatches."""
    import csv
    import glob
    lines = ["# L1/L2 pipeline counters per dispatch (cold-weight benchmark calls), rocprofv3 PMC",
             "# commands (run from /tmp with TMPDIR=/tmp), one run per counter group G and workload W:",
             "#   rocprofv3 --pmc <G> --output-format csv -d ROOT/<W>_g<i> -- python3 bench.py "
             "--traffic-run <W> ; python3 bench.py --summarize-pipeline ROOT"]
    for i, grp in enumerate(PIPELINE_GROUPS):
        lines.append("# group %d: [%s]" % (i, grp))
    lines.append("# values are means over the dispatches of the run; *_sum counters are summed over "
                 "all CUs / L2 channels")
    lines.append("kernel_source_hash: %s" % kernel_source_hash())
    for wl in PIPELINE_WORKLOADS:
        vals = {}
        for i in range(len(PIPELINE_GROUPS)):
            d = os.path.join(root, "%s_g%d" % (wl, i))
            for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
                with open(path) as fh:
                    for r in csv.DictReader(fh):
                        if "w8a16" not in r["Kernel_Name"]:
                            continue
                        name = r["Kernel_Name"].replace("void ", "").replace(
                            "w8a16::(anonymous namespace)::", "").split("(")[0]
                        vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                            float(r["Counter_Value"]))
        lines.append("")
        lines.append("workload %s" % wl)
        for kern in sorted(vals):
            lines.append("  kernel %s" % kern)
            for cname in sorted(vals[kern]):
                v = vals[kern][cname]
                lines.append("    %-36s %.4g" % (cname, sum(v) / len(v)))
    path = os.path.join(ROOT, "profiles", "memory_pipeline_counters.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(open(path).read())


MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE"
CUS = 256              # MI355X
SIMDS = 1024           # 4 per CU
XCDS = 8


def summarize_mfma(pmc_dir: str, wl_name: str):
    """Writes profiles/mfma_<workload>.txt from one rocprofv3 --pmc run of
    MFMA_COUNTERS over a --traffic-run of the workload: per GEMM kernel, the
    MFMA-busy share of SIMD cycles (sum of SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE x SIMDs, the MfmaUtil expression of rocprofiler-sdk's
    counter definitions) and the BF16 MFMA work it counted (MOPS x 512 =
    flops) against 2*M*N*K."""
    import csv
    import glob
    import datagen
    wl = datagen.workload(wl_name)
    vals = {}
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if "w8a16" not in r["Kernel_Name"]:
                    continue
                name = r["Kernel_Name"].replace("void ", "").replace(
                    "w8a16::(anonymous namespace)::", "").split("(")[0]
                vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    path = os.path.join(ROOT, "profiles", "mfma_%s.txt" % wl.name)
    with open(path, "w") as fh:
        fh.write("# MFMA utilisation per GEMM dispatch on workload %s, rocprofv3 PMC\n" % wl.name)
        fh.write("# command (run from /tmp with TMPDIR=/tmp):\n#   rocprofv3 --pmc %s "
                 "--output-format csv -d PMC_DIR -- python3 bench.py --traffic-run %s ; "
                 "python3 bench.py --summarize-mfma PMC_DIR %s\n" % (MFMA_COUNTERS, wl.name, wl.name))
        fh.write("# values are means over the run's dispatches; rocprofv3 sums GRBM_GUI_ACTIVE over "
                 "the %d XCDs and SQ_VALU_MFMA_BUSY_CYCLES over the %d SIMDs, so\n" % (XCDS, SIMDS))
        fh.write("#   mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d * %d)   "
                 "(rocprofiler-sdk's MfmaUtil, with the max over XCDs as the mean)\n" % (XCDS, SIMDS))
        fh.write("#   mfma_util_cu_busy = (SQ_VALU_MFMA_BUSY_CYCLES / %d) / (SQ_BUSY_CU_CYCLES / %d)  "
                 "(MFMA-busy share of the cycles the CUs were busy)\n" % (SIMDS, CUS))
        fh.write("kernel_source_hash: %s\n" % kernel_source_hash())
        fh.write("flops_per_call: %d\n" % wl.flops())
        for k in sorted(vals):
            v = {c: sum(x) / len(x) for c, x in vals[k].items()}
            busy, active = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), v.get("GRBM_GUI_ACTIVE", 0.0)
            cu_busy = v.get("SQ_BUSY_CU_CYCLES", 0.0)
            util = busy / (active / XCDS * SIMDS) if active else float("nan")
            util_cu = (busy / SIMDS) / (cu_busy / CUS) if cu_busy else float("nan")
            mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
            fh.write("kernel %s: dispatches %d, " % (k, len(next(iter(vals[k].values())))) +
                     ", ".join("%s %.6g" % (c, x) for c, x in sorted(v.items())) +
                     ", mfma_util %.4f, mfma_util_cu_busy %.4f, bf16_mfma_flops %.6g\n"
                     % (util, util_cu, mops * 512))
    print(open(path).read())


def summarize_traffic(fetch_dir: str, write_dir: str, wl_name: str, command: str):
    """Writes profiles/traffic_<workload>.txt: HBM bytes per launch of the
    GEMM kernel(s) from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for one plain device copy of
    COPY_BYTES (the largest copy dispatch of the run)."""
    import datagen
    wl = datagen.workload(wl_name)
    fetch = _pmc_values(fetch_dir, "FETCH_SIZE")
    write = _pmc_values(write_dir, "WRITE_SIZE")
    copy_kib = COPY_BYTES / 1024.0

    def copy_max(vals):
        # torch's device-to-device copy_ of a contiguous tensor is a runtime
        # buffer copy; the arena's replica copies are elementwise kernels
        best = 0.0
        for k, v in vals.items():
            if "copyBuffer" in k:
                best = max(best, max(v))
        return best

    cw = copy_max(write)                 # the copy writes exactly what it copies
    cf = copy_max(fetch)
    f_scale = copy_kib / cf if cf > 0 else float("nan")
    w_scale = copy_kib / cw if cw > 0 else float("nan")
    lines = []
    total = 0.0
    kernels = sorted(k for k in fetch if "w8a16" in k)
    for k in kernels:
        f = sum(fetch[k]) / len(fetch[k])
        w = sum(write.get(k, [0.0])) / max(1, len(write.get(k, [])))
        b = (f * f_scale + w * w_scale) * 1024.0
        total += b
        lines.append((k, len(fetch[k]), f, w, b))
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % wl.name)
    with open(path, "w") as fh:
        fh.write("# HBM traffic per GEMM call on workload %s, from rocprofv3 PMC counters\n"
                 % wl.name)
        fh.write("# commands (run from /tmp with TMPDIR=/tmp):\n#   %s\n" % command)
        fh.write("kernel_source_hash: %s\n" % kernel_source_hash())
        fh.write("copy_bytes: %d\n" % COPY_BYTES)
        fh.write("copy_fetch_kib_raw: %.1f\n" % cf)
        fh.write("copy_write_kib_raw: %.1f\n" % cw)
        fh.write("fetch_scale: %.4f\n" % f_scale)
        fh.write("write_scale: %.4f\n" % w_scale)
        for k, n, f, w, b in lines:
            short = k.replace("void ", "").replace("w8a16::(anonymous namespace)::", "")
            short = short.split("(")[0]
            fh.write("kernel %s: dispatches %d, fetch_kib_raw %.1f, write_kib_raw %.1f, "
                     "hbm_bytes %.0f\n" % (short, n, f, w, b))
        fh.write("hbm_bytes_per_launch: %.0f\n" % total)
        fh.write("algorithmic_bytes_per_launch: %d\n" % wl.algorithmic_bytes())
        fh.write("traffic_over_algorithmic: %.3f\n" % (total / wl.algorithmic_bytes()))
    print(open(path).read())


def summarize_trace(trace_dir: str, wl_name: str, command: str, last: int = 0):
    """Writes profiles/kernel_trace_<workload>.txt from a rocprofv3
    --kernel-trace --stats run: per-kernel dispatch counts and durations.
    last > 0 keeps only each kernel's `last` latest dispatches (the timed
    graph replay of a --trace-run), and also gives the span from the first
    to the last of them per dispatch (the time per call the replay saw)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as fh:
            rows.extend(csv.DictReader(fh))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    path = os.path.join(ROOT, "profiles", "kernel_trace_%s.txt" % wl_name)
    spans = []
    with open(path, "w") as fh:
        fh.write("# rocprofv3 kernel trace of the benchmark on workload %s\n" % wl_name)
        fh.write("# command (run from /tmp with TMPDIR=/tmp):\n#   %s\n" % command)
        fh.write("kernel_source_hash: %s\n" % kernel_source_hash())
        if last:
            fh.write("# each kernel's last %d dispatches: the timed graph replay\n" % last)
        fh.write("# kernel | dispatches | mean_us | median_us | min_us | max_us\n")
        for k, ts in sorted(by.items(), key=lambda kv: -len(kv[1])):
            if "w8a16" not in k:
                continue
            ts = sorted(ts)
            if last:
                ts = ts[-last:]
                spans.append((ts[0][0], ts[-1][1]))
            ds = sorted((e - b) / 1000.0 for b, e in ts)
            short = k.replace("void ", "").replace("w8a16::(anonymous namespace)::", "")
            fh.write("%s | %d | %.3f | %.3f | %.3f | %.3f\n" % (
                short, len(ds), sum(ds) / len(ds), ds[len(ds) // 2], ds[0], ds[-1]))
        if spans and last:
            b = min(x[0] for x in spans)
            e = max(x[1] for x in spans)
            fh.write("replay_span_us_per_call: %.3f\n" % ((e - b) / 1000.0 / last))
    print(open(path).read())


M_SWEEP = [1, 2, 4, 8, 12, 16, 24, 32, 40, 48, 56, 64, 65, 80, 96, 112, 128, 160, 192, 256]


def m_sweep(n: int, k: int, steps: int = 50):
    """Default plan over the row counts of M_SWEEP at one (n, k): one JSON
    line per m (cold weights, graph replay)."""
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    w8.library()
    for m in M_SWEEP:
        prob = datagen.make_problem(m, n, k, seed=7000 + m)
        plan = w8.plan(m, n, k, torch.cuda.get_device_properties(0).multi_processor_count)
        # one untimed pass first: the first timing of a fresh arena runs slow
        ar, _, _, _ = time_workload(torch, w8, prob, 10, 3)
        del ar
        arena, ms, eager_ms, replicas = time_workload(torch, w8, prob, steps, 5)
        ok = check_arena_output(arena, steps + 5)
        del arena
        torch.cuda.empty_cache()
        nbytes = n * k + 4 * (-(-n // 128)) * (k // 128) + 2 * m * k + 2 * m * n
        print(json.dumps({"m": m, "n": n, "k": k, "us_per_call": round(ms * 1e3, 3),
                          "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "tflops": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 2),
                          "kernel": {w8.KERNEL_STREAM: "stream", w8.KERNEL_TILE: "tile",
                                     w8.KERNEL_RING: "ring"}.get(plan.kernel, "?"),
                          "plan": plan.as_dict(), "output_sane": ok}), flush=True)


QKV_ARMS = (4096, 1024, 1024)      # Q, K, V output widths (grouped K/V heads)


def batched_bench(m: int = 8, k: int = 4096, steps: int = 100, warmup: int = 10):
    """The batched tier on decode-size Q/K/V arms sharing one A (m rows,
    hidden k): one w8a16_gemm_batched call per step against the same arms
    as three w8a16_gemm calls, both cold (replicas over >= 512 MiB) and in
    graph replay.  Prints one JSON line."""
    import numpy as np
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    w8.library()
    probs = [datagen.make_problem(m, n, k, seed=8000 + i) for i, n in enumerate(QKV_ARMS)]
    per = probs[0].a.nbytes + sum(p.w.nbytes + p.scale.nbytes + p.c.nbytes for p in probs)
    reps = max(1, -(-ARENA_BYTES // per))
    dev = torch.device("cuda")
    a = torch.from_numpy(probs[0].a).view(torch.int16).to(dev).reshape(1, -1).repeat(reps, 1)
    arms = []
    for p in probs:
        w = torch.from_numpy(p.w).to(dev).reshape(1, -1).repeat(reps, 1)
        sc = torch.from_numpy(p.scale).to(dev).reshape(1, -1).repeat(reps, 1)
        c = torch.from_numpy(p.c).view(torch.int16).to(dev).reshape(1, -1).repeat(reps, 1)
        arms.append((p, w, sc, c))

    def descs(i):
        r = i % reps
        return [dict(a=a[r].data_ptr(), w_fp8=w[r].data_ptr(), block_scale=sc[r].data_ptr(),
                     c=c[r].data_ptr(), a_row_stride=k, c_row_stride=p.n, m=m, n=p.n, k=k)
                for (p, w, sc, c) in arms]

    stream = torch.cuda.Stream()

    def batched(i):
        st = w8.gemm_batched_raw(descs(i), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(w8.last_error())

    def separate(i):
        for d in descs(i):
            st = w8.gemm_raw(d["a"], k, d["w_fp8"], d["block_scale"], d["c"], d["n"], m,
                             d["n"], k, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(w8.last_error())

    def graph_ms(fn):
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    fn(warmup + i)
            g.replay()
            torch.cuda.synchronize()
            start.record(stream)
            g.replay()
            stop.record(stream)
            torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    ms_sep = graph_ms(separate)
    ms_b = graph_ms(batched)
    ok = True
    for (p, w, sc, c) in arms:
        for r in range(min(reps, steps + warmup)):
            cc = c[r].cpu().numpy().view(np.uint16).reshape(p.c.shape)
            ok &= bool(((cc[:m, :p.n] & 0x7F80) != 0x7F80).all())
    nbytes = sum(p.n * k + 4 * (-(-p.n // 128)) * (k // 128) + 2 * m * k + 2 * m * p.n
                 for p in probs)
    flops = sum(2.0 * m * p.n * k for p in probs)
    plan = w8.plan_batched([(m, n, k) for n in QKV_ARMS],
                           torch.cuda.get_device_properties(0).multi_processor_count)
    gbs = nbytes / (ms_b * 1e-3) / 1e9
    print(json.dumps({
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms_b, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qkv_batched_m%d_k%d_n%s" % (m, k, "_".join(map(str, QKV_ARMS))),
                   "m": m, "k": k, "arms_n": list(QKV_ARMS), "shared_a": True,
                   "weights": "cold", "arena_replicas": reps},
        "us_per_call": round(ms_b * 1e3, 3),
        "us_per_call_separate_calls": round(ms_sep * 1e3, 3),
        "speedup_vs_separate": round(ms_sep / ms_b, 3),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tflops": round(flops / (ms_b * 1e-3) / 1e12, 3),
        "plan": plan.as_dict(), "output_sane": ok,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "w8a16_stream_batched_kernel",
                     "algorithmic_bytes_per_launch": nbytes},
        "kernel_source_hash": kernel_source_hash(), "note": NOTE}), flush=True)


def time_graph(torch, stream, call, steps: int, warmup: int, scrub=None):
    """(graph ms per call, eager ms per call) of call(0..steps-1) on
    `stream`, with the spin-up and cache scrub of time_workload before each
    timed region."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                call(i)

        def spin_up():
            t0 = time.perf_counter()
            while True:
                graph.replay()
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= SPIN_UP_S:
                    break
            if scrub is not None:
                scrub.run()

        spin_up()
        start.record(stream)
        for i in range(steps):
            call(i)
        stop.record(stream)
        torch.cuda.synchronize()
        eager_ms = start.elapsed_time(stop) / steps
        spin_up()
        start.record(stream)
        graph.replay()
        stop.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, eager_ms


# (m, n, k, A row pitch in elements): the W8A16 workloads' shapes, and a
# wide weight (2048 16-row tiles) that the persistent kernel serves.
W4A4_WORKLOADS = [(8, 4096, 4096, 4096), (16, 12288, 5120, 5120), (32, 6144, 2048, 2560),
                  (16, 32768, 4096, 4096)]


def w4a4_bench(steps: int = 100, warmup: int = 10):
    """The W4A4 MX GEMV on its workloads, cold (replicas over >= 512 MiB,
    cache scrub, graph replay).  One JSON line per workload."""
    import numpy as np
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    w8.library()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    scrub = Scrub(torch)
    for m, n, k, pitch in W4A4_WORKLOADS:
        p = datagen.make_mx_problem(m, n, k, seed=9000 + m + n + k, a_row_stride=pitch)
        per = p.a.nbytes + p.a_scale.nbytes + p.w.nbytes + p.w_scale.nbytes + 2 * m * n
        reps = max(1, -(-ARENA_BYTES // per))
        dev = torch.device("cuda")

        def rep(x):
            return torch.from_numpy(np.ascontiguousarray(x)).to(dev).reshape(1, -1).repeat(reps, 1)

        a, asc, w, wsc = rep(p.a), rep(p.a_scale), rep(p.w), rep(p.w_scale)
        c = torch.zeros((reps, m * n), dtype=torch.int16, device=dev)
        stream = torch.cuda.Stream()

        def call(i):
            r = i % reps
            st = w8.gemm_w4a4_raw(a[r].data_ptr(), pitch, asc[r].data_ptr(), w[r].data_ptr(),
                                  wsc[r].data_ptr(), c[r].data_ptr(), n, m, n, k,
                                  stream.cuda_stream)
            if st != 0:
                raise RuntimeError(w8.last_error())

        ms, eager = time_graph(torch, stream, call, steps, warmup, scrub)
        ok = True
        for r in range(min(reps, steps)):
            cc = c[r].cpu().numpy().view(np.uint16)
            ok &= bool(((cc & 0x7F80) != 0x7F80).all())
        nbytes = p.algorithmic_bytes()
        gbs = nbytes / (ms * 1e-3) / 1e9
        plan = w8.plan_w4a4(m, n, k, cus)
        kname = "w8a16_w4a4_ps_kernel" if plan.kernel == w8.KERNEL_W4A4_PS else "w8a16_w4a4_kernel"
        print(json.dumps({
            "metric": METRIC_W4A4, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp4", "data": "synthetic",
            "config": {"workload": "w4a4_m%d_n%d_k%d" % (m, n, k), "m": m, "n": n, "k": k,
                       "a_row_stride": pitch, "format": "MXFP4 (E2M1, E8M0 per 32)",
                       "weights": "cold", "arena_replicas": reps},
            "us_per_call": round(ms * 1e3, 3), "us_per_call_eager": round(eager * 1e3, 3),
            "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "tflops": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 3),
            "plan": plan.as_dict(), "output_sane": ok,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": kname, "algorithmic_bytes_per_launch": nbytes},
            "kernel_source_hash": kernel_source_hash(), "note": NOTE}), flush=True)
        del a, asc, w, wsc, c
        torch.cuda.empty_cache()


W8A8_WORKLOADS = ["m8_n4096_k4096", "m16_n12288_k5120", "m32_n6144_k2048_strided"]


def w8a8_bench(steps: int = 100, warmup: int = 10):
    """The FP8-activation path on the workloads' shapes (contiguous pitches):
    the quantizer alone, the W8A8 GEMM alone and both back to back, each
    cold (replicas over >= 512 MiB) in graph replay.  One JSON line per
    workload."""
    import numpy as np
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    w8.library()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for name in W8A8_WORKLOADS:
        wl = datagen.workload(name)
        m, n, k = wl.m, wl.n, wl.k
        p = datagen.make_problem(m, n, k, seed=wl.seed)
        per = 2 * m * k + m * k + 4 * m * (k // 128) + p.w.nbytes + p.scale.nbytes + 2 * m * n
        reps = max(1, -(-ARENA_BYTES // per))
        dev = torch.device("cuda")
        a = torch.from_numpy(p.a[:, :k].copy()).view(torch.int16).to(dev).reshape(1, -1).repeat(reps, 1)
        q = torch.zeros((reps, m * k), dtype=torch.uint8, device=dev)
        sa = torch.zeros((reps, m * (k // 128)), dtype=torch.float32, device=dev)
        w = torch.from_numpy(p.w).to(dev).reshape(1, -1).repeat(reps, 1)
        sw = torch.from_numpy(p.scale).to(dev).reshape(1, -1).repeat(reps, 1)
        c = torch.zeros((reps, m * n), dtype=torch.int16, device=dev)
        stream = torch.cuda.Stream()

        def quant(i):
            r = i % reps
            st = w8.act_quant_fp8_raw(a[r].data_ptr(), k, q[r].data_ptr(), k, sa[r].data_ptr(),
                                      m, k, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(w8.last_error())

        def gemm(i):
            r = i % reps
            st = w8.gemm_w8a8_raw(q[r].data_ptr(), k, sa[r].data_ptr(), w[r].data_ptr(),
                                  sw[r].data_ptr(), c[r].data_ptr(), n, m, n, k,
                                  stream.cuda_stream)
            if st != 0:
                raise RuntimeError(w8.last_error())

        def both(i):
            quant(i)
            gemm(i)

        def graph_ms(fn):
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                for i in range(warmup):
                    fn(i)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(steps):
                        fn(warmup + i)
                g.replay()
                torch.cuda.synchronize()
                start.record(stream)
                g.replay()
                stop.record(stream)
                torch.cuda.synchronize()
            return start.elapsed_time(stop) / steps

        ms_both = graph_ms(both)
        ms_q = graph_ms(quant)
        ms_g = graph_ms(gemm)
        ok = True
        for r in range(min(reps, steps + warmup)):
            cc = c[r].cpu().numpy().view(np.uint16)
            ok &= bool(((cc & 0x7F80) != 0x7F80).all())
        g_bytes = n * k + 4 * (-(-n // 128)) * (k // 128) + m * k + 4 * m * (k // 128) + 2 * m * n
        q_bytes = 2 * m * k + m * k + 4 * m * (k // 128)
        gbs = g_bytes / (ms_g * 1e-3) / 1e9
        plan = w8.plan_w8a8(m, n, k, cus)
        print(json.dumps({
            "metric": METRIC_W8A8, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": ms_g, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
            "config": {"workload": "w8a8_" + name, "m": m, "n": n, "k": k, "weights": "cold",
                       "arena_replicas": reps},
            "us_per_call": round(ms_g * 1e3, 3),
            "us_quantizer": round(ms_q * 1e3, 3),
            "us_quantizer_plus_gemm": round(ms_both * 1e3, 3),
            "quantizer_gbs": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "tflops": round(2.0 * m * n * k / (ms_g * 1e-3) / 1e12, 3),
            "plan": plan.as_dict(), "output_sane": ok,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "w8a16_w8a8_kernel", "algorithmic_bytes_per_launch": g_bytes},
            "kernel_source_hash": kernel_source_hash(), "note": NOTE}), flush=True)
        del a, q, sa, w, sw, c
        torch.cuda.empty_cache()


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--w4a4":
        w4a4_bench()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--w8a8":
        w8a8_bench()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--batched":
        batched_bench()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--m-sweep":
        n = int(sys.argv[2]) if len(sys.argv) > 2 else 8192
        k = int(sys.argv[3]) if len(sys.argv) > 3 else 8192
        m_sweep(n, k)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-run":
        trace_run(sys.argv[2] if len(sys.argv) > 2 else MAIN_WORKLOAD,
                  int(sys.argv[3]) if len(sys.argv) > 3 else 20)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        wl_name = sys.argv[3] if len(sys.argv) > 3 else MAIN_WORKLOAD
        if wl_name in ("batched", "w8a8", "w4a4"):      # the --batched / --w8a8 / --w4a4 legs
            cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d TRACE_DIR -- "
                   "python3 bench.py --%s ; python3 bench.py --summarize-trace TRACE_DIR %s"
                   % (wl_name, wl_name))
            summarize_trace(sys.argv[2], wl_name, cmd)
        else:
            steps = int(sys.argv[4]) if len(sys.argv) > 4 else 20
            cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d TRACE_DIR -- "
                   "python3 bench.py --trace-run %s %d ; "
                   "python3 bench.py --summarize-trace TRACE_DIR %s %d"
                   % (wl_name, steps, wl_name, steps))
            summarize_trace(sys.argv[2], wl_name, cmd, last=steps)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-mfma":
        summarize_mfma(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else "m128_n8192_k8192")
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pipeline":
        summarize_pipeline(sys.argv[2])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-run":
        traffic_run(sys.argv[2] if len(sys.argv) > 2 else MAIN_WORKLOAD)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-traffic":
        wl_name = sys.argv[4] if len(sys.argv) > 4 else MAIN_WORKLOAD
        cmd = ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d FETCH_DIR -- python3 "
               "bench.py --traffic-run %s ; rocprofv3 --pmc WRITE_SIZE --output-format csv "
               "-d WRITE_DIR -- python3 bench.py --traffic-run %s ; python3 bench.py "
               "--summarize-traffic FETCH_DIR WRITE_DIR %s" % (wl_name, wl_name, wl_name))
        summarize_traffic(sys.argv[2], sys.argv[3], wl_name, cmd)
        return
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

    import numpy as np
    import torch

    import block_scaled_fp8_w8a16_amd as w8
    import datagen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w8.library()
    khash = kernel_source_hash()

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    scrub = None if args.warm else Scrub(torch)

    def measure(w, steps, warmup):
        """Times one workload; keeps a host copy of the C written by call 0
        (replica 0) for the CPU leg's check against the oracle."""
        log("generating %s" % w.name)
        pr = datagen.make_workload(w)
        pl = w8.plan(w.m, w.n, w.k, cus)
        log("timing %s plan=%s" % (w.name, pl.as_dict()))
        ar, ms, eager, reps = time_workload(torch, w8, pr, steps, warmup, cold=not args.warm,
                                            scrub=scrub)
        ok = check_arena_output(ar, steps)
        c0 = ar.c[0].cpu().numpy().view(np.uint16).reshape(pr.c.shape).copy()
        per = pr.a.nbytes + pr.w.nbytes + pr.scale.nbytes + pr.c.nbytes
        del ar
        torch.cuda.empty_cache()
        warm_ms = None
        if not args.warm:
            # context only: the same buffers on every call, so the weight
            # may be served from the Infinity Cache
            ar_w, warm_ms, _, _ = time_workload(torch, w8, pr, steps, warmup, cold=False)
            del ar_w
            torch.cuda.empty_cache()
        gb = w.algorithmic_bytes() / (ms * 1e-3) / 1e9
        tf = w.flops() / (ms * 1e-3) / 1e12
        log("%s: %.3f us/call, %.1f GB/s, %.1f TFLOP/s (output sane %s)" %
            (w.name, ms * 1e3, gb, tf, ok))
        row = {"workload": w.name, "us_per_call": round(ms * 1e3, 3),
               "us_per_call_eager": round(eager * 1e3, 3),
               "gbs": round(gb, 1), "pct_hbm": round(100 * gb / HBM_PEAK_GBS, 2),
               "tflops": round(tf, 3), "pct_mfma": round(100 * tf / BF16_PEAK_TFLOPS, 2),
               "output_sane": ok, "plan": pl.as_dict(), "arena_replicas": reps,
               "timed_distinct_replica_bytes": min(steps, reps) * per, "seed": w.seed}
        if warm_ms is not None:
            row["us_per_call_warm"] = round(warm_ms * 1e3, 3)
            row["gbs_warm"] = round(w.algorithmic_bytes() / (warm_ms * 1e-3) / 1e9, 1)
        return pr, pl, ms, eager, reps, ok, c0, row

    wl = datagen.workload(args.workload)
    prob, plan, ms_call, eager_ms, replicas, sane, c_main, main_row = measure(
        wl, args.steps, args.warmup)
    alg_bytes = wl.algorithmic_bytes()
    gbs = alg_bytes / (ms_call * 1e-3) / 1e9
    checked = [(wl, prob, c_main, main_row)]

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
                   "arena_replicas": replicas,
                   "timed_distinct_replica_bytes": main_row["timed_distinct_replica_bytes"],
                   "cache_scrub_bytes": 0 if args.warm else SCRUB_BYTES},
        "us_per_call": round(ms_call * 1e3, 3),
        "us_per_call_eager": round(eager_ms * 1e3, 3),
        "us_per_call_warm": main_row.get("us_per_call_warm"),
        "timing": ("HIP graph of the K calls, replayed once; HIP events on the launch stream; "
                   "before it ~20 ms of untimed replays (working clock) and a 512 MiB fill "
                   "that evicts the Infinity Cache; call i reads replica i mod R; "
                   "us_per_call_warm: the same on one set of buffers, after the cold timing "
                   "(the weight may stay in the Infinity Cache), context only"),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "peaks": {"hbm_gbs": HBM_PEAK_GBS, "bf16_dense_tflops": BF16_PEAK_TFLOPS,
                  "source": "published MI355X figures (HBM3E 8 TB/s; dense BF16 MFMA "
                            "2.5 PFLOP/s), the denominators of pct_hbm and pct_mfma"},
        "tflops": round(wl.flops() / (ms_call * 1e-3) / 1e12, 3),
        "plan": plan.as_dict(),
        "output_sane": sane,
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": {w8.KERNEL_STREAM: "w8a16_stream_kernel", w8.KERNEL_TILE: "w8a16_tile_kernel",
                       w8.KERNEL_RING: "w8a16_ring_kernel"}.get(plan.kernel, "?"),
            "algorithmic_bytes_per_launch": alg_bytes,
        },
        "kernel_source_hash": khash,
        "note": NOTE,
    }

    if not args.only_main:
        rows = []
        for other in datagen.WORKLOADS:
            if other.name == wl.name:
                rows.append(main_row)
                continue
            steps = max(20, min(args.steps, 200))
            owarm = max(5, args.warmup // 2)
            op, _, _, _, _, _, oc0, orow = measure(other, steps, owarm)
            rows.append(orow)
            checked.append((other, op, oc0, orow))
        result["all_workloads"] = rows

    if not args.no_cpu:
        import oracle   # the CPU baseline leg is the only part that runs the oracle
        log("timing the CPU oracle on %s" % wl.name)
        dt, reps, threads = cpu_baseline(oracle, datagen, prob)
        log("timing the CPU oracle on %s, one thread" % wl.name)
        dt1, reps1, _ = cpu_baseline(oracle, datagen, prob, budget_s=5.0, threads=1)
        result["cpu_baseline"] = {
            "value": round(alg_bytes / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "%d whole %s GEMMs (FP64 C oracle, OpenMP, %d threads), %.3f s each" %
                      (reps, wl.name, threads, dt),
            "us_per_call": round(dt * 1e6, 1),
            "single_thread": {"value": round(alg_bytes / dt1 / 1e9, 4), "unit": "GB/s",
                              "us_per_call": round(dt1 * 1e6, 1),
                              "sample": "%d whole GEMMs, 1 thread" % reps1},
        }
        # The same leg grades what each timed workload's call 0 wrote
        # against the whole oracle (a diagnostic; parity itself is the GPU
        # tests' job).
        for w, pr, c0, row in checked:
            log("oracle check of %s" % w.name)
            row["oracle_check"] = oracle_check(oracle, pr, c0, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
