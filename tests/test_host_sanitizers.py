"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner (``plan.cpp``: argument checks, default plans, caller-edited
plans, batched plans, status and error strings) and the CPU oracle (both C
files) are rebuilt with ``-fsanitize=address,undefined`` and driven by the
small programs under ``tests/host/``: sweeps of shapes, random edits of
plans, and operands allocated to exactly their documented extent.  Any
sanitizer report aborts the program (``-fno-sanitize-recover=all``); the
drivers also check the invariants of every plan the planner accepts.  The
GPU kernels are not built here (no GPU sanitizer on this hardware)."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "block_scaled_fp8_w8a16_amd", "csrc")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe, expect):
    build = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True, timeout=240)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=240, env=ENV)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert expect in run.stdout and "ok" in run.stdout, run.stdout
    assert "runtime error" not in run.stderr, run.stderr[-4000:]
    return run.stdout


def test_planner_under_asan_ubsan(tmp_path):
    out = _build_and_run(
        ["g++", "-std=c++17"] + SAN + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                       os.path.join(CSRC, "plan.cpp"),
                                       os.path.join(HOST, "sanitize_plan.cpp")],
        str(tmp_path / "sanitize_plan"), "planner sweep done")
    accepted = int(out.split("(")[1].split()[0])
    assert accepted > 10000, out     # the edits reach accepted plans, not only rejections


def test_oracle_under_asan_ubsan(tmp_path):
    _build_and_run(
        ["gcc", "-std=c11", "-ffp-contract=off"] + SAN +
        [os.path.join(ROOT, "oracle", "w8a16_oracle.c"),
         os.path.join(ROOT, "oracle", "w4a4_oracle.c"),
         os.path.join(HOST, "sanitize_oracle.c"), "-lm"],
        str(tmp_path / "sanitize_oracle"), "oracle sweep done")
