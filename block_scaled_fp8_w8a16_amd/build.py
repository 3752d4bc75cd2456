"""Build ``libw8a16.so`` (the HIP kernels and their C ABI) for gfx950.

Run as ``python -m block_scaled_fp8_w8a16_amd.build``.  The library is built
in-tree next to this file so it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libw8a16.so")

SOURCES = ["plan.cpp", "api.hip", "stream_kernel.hip", "tile_m64.hip", "tile_m128.hip",
           "wide_kernel.hip", "split_reduce.hip", "ring_kernel.hip", "w8a8_kernel.hip",
           "w4a4_kernel.hip"]
HEADERS = ["plan.h", "kernels.h", "device_common.h", "tile_kernel.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed FP32 ops (v_pk_*_f32) are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Per-source extras.  The tile kernel folds each K step's MFMA partial into
# FP32 accumulators with VALU FMAs; with the partials in AGPRs every fold
# first copies them out (v_accvgpr_read), which measured as the single most
# expensive part of its loop.  The VGPR form of the MFMA keeps them in VGPRs.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"tile_m64.hip": _VGPR_FORM, "tile_m128.hip": _VGPR_FORM,
               "w8a8_kernel.hip": _VGPR_FORM}


def _compile_cmd(src: str, obj: str) -> list:
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        return [HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Wall", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS + \
               EXTRA_FLAGS.get(src, []) + ["-c", path, "-o", obj]
    return ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
            "-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, at most 8 at a time) and link."""
    builddir = os.path.join(HERE, "_build")
    os.makedirs(builddir, exist_ok=True)
    objs = [os.path.join(builddir, src + ".o") for src in SOURCES]
    cmds = [_compile_cmd(src, obj) for src, obj in zip(SOURCES, objs)]
    if verbose:
        for cmd in cmds:
            print(" ".join(cmd), flush=True)
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for fut in [pool.submit(subprocess.run, cmd, check=True) for cmd in cmds]:
            fut.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
