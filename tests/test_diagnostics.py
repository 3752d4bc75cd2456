"""The diagnostic environment variables W8A16_LOG and W8A16_DEBUG_SYNC.

They are read once per process, so every case runs a child process.  The
CPU cases need no GPU: a bad value is rejected before any other check or
GPU call, and the pure planning calls ignore the variables.  The GPU case
runs every enqueuing entry point with both on, checks the log (one line per
distinct launch, the planner's reason, the caller's plan marked as such)
and that the outputs equal those of the same calls made without them."""

import os
import subprocess
import sys

import numpy as np
import pytest

import block_scaled_fp8_w8a16_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _child(code, **env):
    e = dict(os.environ)
    for key in ("W8A16_LOG", "W8A16_DEBUG_SYNC"):
        e.pop(key, None)
    e.update(env)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=e, capture_output=True,
                          text=True, timeout=300)


_BAD_VALUE = """
import block_scaled_fp8_w8a16_amd as w8
print(w8.gemm_raw(1, 128, 2, 3, 4, 16, 1, 16, 128))
print(w8.gemm_raw(1, 128, 2, 3, 4, 16, 0, 16, 128))      # m=0: the setting is checked first
print(w8.gemm_noalloc_raw(1, 128, 2, 3, 4, 16, 1, 16, 128))
print(w8.act_quant_fp8_raw(1, 128, 2, 128, 3, 1, 128))
print(w8.gemm_w8a8_raw(1, 128, 2, 3, 4, 5, 16, 1, 16, 128))
print(w8.gemm_w4a4_raw(1, 128, 2, 3, 4, 5, 16, 1, 16, 128))
print(w8.gemm_batched_raw([dict(a=1, w_fp8=2, block_scale=3, c=4, a_row_stride=128,
                                c_row_stride=16, m=1, n=16, k=128)]))
print(repr(w8.last_error()))
print(w8.plan(16, 4096, 4096).kernel)                     # planning ignores it
"""


@pytest.mark.parametrize("var,value", [("W8A16_LOG", "yes"), ("W8A16_DEBUG_SYNC", "2"),
                                       ("W8A16_LOG", "10")])
def test_bad_setting_fails_every_enqueuing_call(var, value):
    r = _child(_BAD_VALUE, **{var: value})
    assert r.returncode == 0, r.stderr[-3000:]
    lines = r.stdout.split("\n")
    assert lines[:7] == [str(w8.ERR_ENV)] * 7, r.stdout
    assert var in lines[7] and value in lines[7] and "must be 0 or 1" in lines[7]
    assert lines[8] == str(w8.KERNEL_STREAM)
    assert r.stderr == ""


def test_status_string_of_bad_setting():
    assert "W8A16_LOG" in w8.status_string(w8.ERR_ENV)


@pytest.mark.parametrize("value", ["", "0"])
def test_off_values_leave_argument_checks_in_place(value):
    r = _child("import block_scaled_fp8_w8a16_amd as w8\n"
               "print(w8.gemm_raw(1, 128, 2, 3, 4, 16, 0, 16, 128))",
               W8A16_LOG=value, W8A16_DEBUG_SYNC=value)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip() == str(w8.ERR_M_ZERO)
    assert r.stderr == ""


@pytest.mark.gpu
def test_log_and_debug_sync_on_gpu(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    out = tmp_path / "diag.npz"
    print("child: tests/diag_calls.py with W8A16_LOG=1 W8A16_DEBUG_SYNC=1", flush=True)
    r = _child("import runpy, sys; sys.argv = ['diag_calls', %r]; "
               "runpy.run_path('tests/diag_calls.py', run_name='__main__')" % str(out),
               W8A16_LOG="1", W8A16_DEBUG_SYNC="1")
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    log = [ln for ln in r.stderr.split("\n") if ln.startswith("w8a16: ")]

    def lines(prefix):
        return [ln for ln in log if ln.startswith("w8a16: " + prefix)]

    stream = lines("w8a16_gemm m=16 n=4096 k=1024:")
    assert len(stream) == 1, log          # two calls, one line (the graph's call is the same)
    assert "kernel=stream" in stream[0] and "stream kernel" in stream[0]
    split = lines("w8a16_gemm m=1 n=1024 k=8192:")
    assert len(split) == 1 and "K split" in split[0] and "splits=1 " not in split[0], log
    tile = lines("w8a16_gemm m=40 n=2304 k=8192:")
    assert len(tile) == 1 and "kernel=tile" in tile[0], log
    planned = lines("w8a16_gemm_planned m=16 n=4096 k=1024:")
    assert len(planned) == 1 and planned[0].endswith("caller's plan") and \
        "tile=16x32" in planned[0], log
    assert len(lines("w8a16_act_quant_fp8 m=8 k=1024:")) == 1, log
    assert len(lines("w8a16_gemm_w8a8 m=8 n=2048 k=1024: kernel=w8a8")) == 1, log
    w4 = lines("w8a16_gemm_w4a4 m=8 n=4096 k=2048:")
    assert len(w4) == 1 and "W4A4" in w4[0], log
    assert len(lines("w8a16_gemm_batched (2 problems, the first) m=4 n=1024 k=512:")) == 1, log
    assert len(log) == 8, log

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import diag_calls
    ref = diag_calls.run_all()
    got = np.load(out)
    assert sorted(got.files) == sorted(ref), (got.files, list(ref))
    for name, bits in ref.items():
        assert np.array_equal(got[name], bits), name
