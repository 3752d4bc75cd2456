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
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR   (writes profiles/)
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
    """Returns (arena, graph ms per call, eager ms per call, replicas)."""
    per_replica = (prob.a.nbytes + prob.w.nbytes + prob.scale.nbytes + prob.c.nbytes)
    replicas = max(1, -(-ARENA_BYTES // per_replica)) if cold else 1
    arena = Arena(torch, prob, replicas)
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
        start.record(stream)
        for i in range(steps):
            call(warmup + i)
        stop.record(stream)
        torch.cuda.synchronize()
        eager_ms = start.elapsed_time(stop) / steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                call(warmup + i)
        graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        graph.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        graph_ms = start.elapsed_time(stop) / steps
    return arena, graph_ms, eager_ms, replicas


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


COPY_BYTES = 256 << 20


def traffic_run(wl_name: str):
    """A short run for rocprofv3 --pmc: 20 cold calls of the workload, then
    three plain device copies of COPY_BYTES (the counters' calibration)."""
    import torch
    import block_scaled_fp8_w8a16_amd as w8
    import datagen
    wl = datagen.workload(wl_name)
    prob = datagen.make_workload(wl)
    per = prob.a.nbytes + prob.w.nbytes + prob.scale.nbytes + prob.c.nbytes
    replicas = max(1, -(-ARENA_BYTES // per))
    arena = Arena(torch, prob, replicas)
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
PIPELINE_WORKLOADS = ("m8_n4096_k4096", "m16_n12288_k5120", "m128_n8192_k8192")


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


def summarize_trace(trace_dir: str, wl_name: str, command: str):
    """Writes profiles/kernel_trace_<workload>.txt from a rocprofv3
    --kernel-trace --stats run: per-kernel dispatch counts and durations."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as fh:
            rows.extend(csv.DictReader(fh))
    by = {}
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        by.setdefault(r["Kernel_Name"], []).append(d)
    path = os.path.join(ROOT, "profiles", "kernel_trace_%s.txt" % wl_name)
    with open(path, "w") as fh:
        fh.write("# rocprofv3 kernel trace of the benchmark on workload %s\n" % wl_name)
        fh.write("# command (run from /tmp with TMPDIR=/tmp):\n#   %s\n" % command)
        fh.write("kernel_source_hash: %s\n" % kernel_source_hash())
        fh.write("# kernel | dispatches | mean_us | median_us | min_us | max_us\n")
        for k, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            if "w8a16" not in k:
                continue
            ds = sorted(ds)
            short = k.replace("void ", "").replace("w8a16::(anonymous namespace)::", "")
            fh.write("%s | %d | %.3f | %.3f | %.3f | %.3f\n" % (
                short, len(ds), sum(ds) / len(ds), ds[len(ds) // 2], ds[0], ds[-1]))
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
            "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
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
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        wl_name = sys.argv[3] if len(sys.argv) > 3 else MAIN_WORKLOAD
        if wl_name in ("batched", "w8a8"):       # the --batched / --w8a8 legs
            cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d TRACE_DIR -- "
                   "python3 bench.py --%s ; python3 bench.py --summarize-trace TRACE_DIR %s"
                   % (wl_name, wl_name))
        else:
            cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d TRACE_DIR -- "
                   "python3 bench.py --steps 50 --warmup 5 --no-cpu --only-main --workload %s ; "
                   "python3 bench.py --summarize-trace TRACE_DIR %s" % (wl_name, wl_name))
        summarize_trace(sys.argv[2], wl_name, cmd)
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

    import numpy as np  # noqa: F401
    import torch

    import block_scaled_fp8_w8a16_amd as w8
    import datagen

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
    arena, ms_call, eager_ms, replicas = time_workload(torch, w8, prob, args.steps,
                                                       args.warmup, cold=not args.warm)
    sane = check_arena_output(arena, args.steps + args.warmup)
    del arena
    torch.cuda.empty_cache()
    alg_bytes = wl.algorithmic_bytes()
    gbs = alg_bytes / (ms_call * 1e-3) / 1e9
    log("%s: %.3f us/call, %.1f GB/s (output sane %s)" % (wl.name, ms_call * 1e3, gbs, sane))

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
        "us_per_call_eager": round(eager_ms * 1e3, 3),
        "timing": "HIP graph of the K calls, replayed; HIP events on the launch stream",
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
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
                rows.append({"workload": wl.name, "us_per_call": round(ms_call * 1e3, 3),
                         "us_per_call_eager": round(eager_ms * 1e3, 3),
                             "gbs": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 2),
                             "tflops": result["tflops"],
                             "pct_mfma": round(100 * result["tflops"] / BF16_PEAK_TFLOPS, 2),
                             "output_sane": sane, "plan": plan.as_dict(), "seed": wl.seed})
                continue
            log("generating %s" % other.name)
            op = datagen.make_workload(other)
            oplan = w8.plan(other.m, other.n, other.k)
            steps = max(20, min(args.steps, 200))
            owarm = max(5, args.warmup // 2)
            ar, oms, oeager, orep = time_workload(torch, w8, op, steps, owarm)
            ok = check_arena_output(ar, steps + owarm)
            del ar
            torch.cuda.empty_cache()
            ogbs = other.algorithmic_bytes() / (oms * 1e-3) / 1e9
            otf = other.flops() / (oms * 1e-3) / 1e12
            log("%s: %.3f us/call, %.1f GB/s, %.1f TFLOP/s (output sane %s)" %
                (other.name, oms * 1e3, ogbs, otf, ok))
            rows.append({"workload": other.name, "us_per_call": round(oms * 1e3, 3),
                         "us_per_call_eager": round(oeager * 1e3, 3),
                         "gbs": round(ogbs, 1), "pct_hbm": round(100 * ogbs / HBM_PEAK_GBS, 2),
                         "tflops": round(otf, 3),
                         "pct_mfma": round(100 * otf / BF16_PEAK_TFLOPS, 2),
                         "output_sane": ok, "plan": oplan.as_dict(),
                         "arena_replicas": orep, "seed": other.seed})
            del op
        result["all_workloads"] = rows

    if not args.no_cpu:
        import oracle   # the CPU baseline leg is the only part that runs the oracle
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
