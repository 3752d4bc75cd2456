"""CPU oracle for the block-scaled FP8 W8A16 GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it, and this package imports nothing from
the product.

The arithmetic lives in ``w8a16_oracle.c`` (plain C, IEEE double): an exact
OCP E4M3FN decode, an exact BF16 decode, per-output sums over 128-wide K
blocks with the block's FP32 scale applied once to each block's partial dot
product, and one round-to-nearest-even to BF16 straight from double.  It
follows the page "w8a16_gemm_pipelined_m32.rs": the operand layouts in the
doc comment of ``w8a16_gemm_pipelined_m32_strided``, the one-scale-per-K-step
rule in the doc comment of ``W8A16_M32_K_BLOCK`` and the fold points of the
module doc's "Numerics" paragraph.

It also holds the FP8 activation quantizer and the W8A8 GEMM it feeds
(page "fp8_act_quant.rs": per-token groups of 128 K elements), with the
arithmetic reading stated at their functions, and the W4A4 MX GEMV (page
"w4a4_proj/mx_plan.rs", read as OCP MXFP4) in ``w4a4_oracle.c``.

This module is argument marshalling around that C code, plus the parity
tolerance the GPU result is graded with.

Parity pins: every function here is pinned by ``tests/test_oracle.py``:
closed-form and library witnesses for the decodes and the rounding, brute
force with exact rationals for the GEMMs, invariants, and for the parity
tolerance helpers (``bf16_bits_to_f64``, ``bf16_ulp``, ``within_tolerance``)
torch's BF16 decoding of all 65536 patterns, the gap between consecutive
BF16 values, and hand-built values exactly at and one BF16 step past the
bar, for both signs, at zero and for NaN / Inf.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w8a16_oracle.c")
_SRC_MX = os.path.join(_HERE, "w4a4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

K_BLOCK = 128


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` next to its source (gcc, -O2, no fast-math,
    no FMA contraction, OpenMP over output elements)."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_MX)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, _SRC_MX, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u32 = ctypes.c_uint32
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_w8a16_gemm.argtypes = [u16p, u32, u8p, f32p, u16p, u32,
                                          u32, u32, u32, f64p, f64p,
                                          ctypes.c_int]
        lib.oracle_w8a16_gemm.restype = ctypes.c_int
        lib.oracle_w8a16_gemm_at.argtypes = [u16p, u32, u8p, f32p, u32, u32,
                                             u32, u32p, u32p, ctypes.c_int64,
                                             u16p, f64p, f64p, ctypes.c_int]
        lib.oracle_w8a16_gemm_at.restype = ctypes.c_int
        lib.oracle_e4m3_rne.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_rne.restype = ctypes.c_uint8
        lib.oracle_act_quant.argtypes = [u16p, u32, u32, u32, u8p, u32, f32p]
        lib.oracle_act_quant.restype = ctypes.c_int
        lib.oracle_w8a8_gemm.argtypes = [u8p, u32, f32p, u8p, f32p, u16p, u32, u32, u32,
                                         u32, f64p, f64p, ctypes.c_int]
        lib.oracle_w8a8_gemm.restype = ctypes.c_int
        lib.oracle_w8a8_gemm_at.argtypes = [u8p, u32, f32p, u8p, f32p, u32, u32, u32,
                                            u32p, u32p, ctypes.c_int64, u16p, f64p, f64p,
                                            ctypes.c_int]
        lib.oracle_w8a8_gemm_at.restype = ctypes.c_int
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_w4a4_gemm.argtypes = [u8p, u32, u8p, u8p, u8p, u16p, u32, u32, u32, u32,
                                         f64p, f64p, ctypes.c_int]
        lib.oracle_w4a4_gemm.restype = ctypes.c_int
        lib.oracle_w4a4_gemm_at.argtypes = [u8p, u32, u8p, u8p, u8p, u32, u32, u32, u32p, u32p,
                                            ctypes.c_int64, u16p, f64p, f64p, ctypes.c_int]
        lib.oracle_w4a4_gemm_at.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(arr: np.ndarray, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN byte (NaN for 0x7F and 0xFF)."""
    return _load().oracle_e4m3_value(int(code) & 0xFF)


def bf16_value(bits: int) -> float:
    """Value of one BF16 bit pattern."""
    return _load().oracle_bf16_value(int(bits) & 0xFFFF)


def bf16_rne(x: float) -> int:
    """BF16 bits nearest to the double ``x`` (ties to even), rounded once."""
    return int(_load().oracle_bf16_rne(float(x)))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _check_operands(a, w, scale, m, n, k, a_row_stride):
    assert a.dtype == np.uint16 and w.dtype == np.uint8 and \
        scale.dtype == np.float32
    assert a.flags.c_contiguous and w.flags.c_contiguous and \
        scale.flags.c_contiguous
    assert a.size >= (m - 1) * a_row_stride + k, "A too small for its pitch"
    assert w.size >= n * k, "W too small"
    assert scale.size >= ((n + K_BLOCK - 1) // K_BLOCK) * (k // K_BLOCK)


def gemm(a: np.ndarray, w: np.ndarray, scale: np.ndarray, m: int, n: int,
         k: int, a_row_stride: Optional[int] = None,
         c_row_stride: Optional[int] = None, threads: int = 0,
         c_init: Optional[np.ndarray] = None
         ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Whole GEMM.  ``a`` holds BF16 bits (uint16) with row pitch
    ``a_row_stride`` (default k), ``w`` E4M3 bytes [n, k], ``scale`` float32
    [ceil(n/128), k/128].  Returns (c_bits [m, c_row_stride] uint16,
    tot [m, n] float64, bound [m, n] float64).  Elements of C outside the
    first n columns keep ``c_init`` (zeros by default)."""
    a_row_stride = k if a_row_stride is None else int(a_row_stride)
    c_row_stride = n if c_row_stride is None else int(c_row_stride)
    a = np.ascontiguousarray(a).reshape(-1)
    w = np.ascontiguousarray(w).reshape(-1)
    scale = np.ascontiguousarray(scale, dtype=np.float32).reshape(-1)
    _check_operands(a, w, scale, m, n, k, a_row_stride)
    if c_init is None:
        c = np.zeros((m, c_row_stride), dtype=np.uint16)
    else:
        c = np.array(c_init, dtype=np.uint16).reshape(m, c_row_stride).copy()
    tot = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = _load().oracle_w8a16_gemm(
        _ptr(a, ctypes.c_uint16), a_row_stride, _ptr(w, ctypes.c_uint8),
        _ptr(scale, ctypes.c_float), _ptr(c, ctypes.c_uint16), c_row_stride,
        m, n, k, _ptr(tot, ctypes.c_double), _ptr(bound, ctypes.c_double),
        int(threads))
    if rc != 0:
        raise ValueError("oracle: invalid shape m=%d n=%d k=%d" % (m, n, k))
    return c, tot, bound


def gemm_at(a: np.ndarray, w: np.ndarray, scale: np.ndarray, m: int, n: int,
            k: int, rows: np.ndarray, cols: np.ndarray,
            a_row_stride: Optional[int] = None, threads: int = 0
            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Selected outputs C[rows[s], cols[s]].  Returns (c_bits uint16 [s],
    tot float64 [s], bound float64 [s])."""
    a_row_stride = k if a_row_stride is None else int(a_row_stride)
    a = np.ascontiguousarray(a).reshape(-1)
    w = np.ascontiguousarray(w).reshape(-1)
    scale = np.ascontiguousarray(scale, dtype=np.float32).reshape(-1)
    _check_operands(a, w, scale, m, n, k, a_row_stride)
    rows = np.ascontiguousarray(rows, dtype=np.uint32).reshape(-1)
    cols = np.ascontiguousarray(cols, dtype=np.uint32).reshape(-1)
    assert rows.size == cols.size
    ns = rows.size
    c = np.empty(ns, dtype=np.uint16)
    tot = np.empty(ns, dtype=np.float64)
    bound = np.empty(ns, dtype=np.float64)
    rc = _load().oracle_w8a16_gemm_at(
        _ptr(a, ctypes.c_uint16), a_row_stride, _ptr(w, ctypes.c_uint8),
        _ptr(scale, ctypes.c_float), m, n, k, _ptr(rows, ctypes.c_uint32),
        _ptr(cols, ctypes.c_uint32), ns, _ptr(c, ctypes.c_uint16),
        _ptr(tot, ctypes.c_double), _ptr(bound, ctypes.c_double),
        int(threads))
    if rc != 0:
        raise ValueError("oracle: invalid shape or sample index")
    return c, tot, bound


# ---------------------------------------------------------------------------
# FP8 activation quantizer and W8A8 GEMM (page "fp8_act_quant.rs": per-token
# groups of 128 K elements).  The arithmetic is a reading (the page gives
# only the grouping): s = amax / 448 and code = E4M3 RNE of x / s, both
# divisions in binary32, saturated to +-448; an all-zero group has s = 0.
# ---------------------------------------------------------------------------

def e4m3_rne(x: float) -> int:
    """OCP E4M3FN code nearest to the float32 ``x`` (ties to even,
    saturating, sign of zero kept)."""
    return int(_load().oracle_e4m3_rne(float(np.float32(x))))


def act_quant(a: np.ndarray, m: int, k: int, a_row_stride: Optional[int] = None,
              q_row_stride: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token, per-128-group FP8 quantization of BF16 bits ``a``
    [m, a_row_stride].  Returns (codes uint8 [m, q_row_stride], scales
    float32 [m, k/128]); code columns past k are zero."""
    a_row_stride = k if a_row_stride is None else int(a_row_stride)
    q_row_stride = k if q_row_stride is None else int(q_row_stride)
    a = np.ascontiguousarray(a, dtype=np.uint16).reshape(-1)
    assert a.size >= (m - 1) * a_row_stride + k
    q = np.zeros((m, q_row_stride), dtype=np.uint8)
    s = np.zeros((m, k // K_BLOCK), dtype=np.float32)
    rc = _load().oracle_act_quant(_ptr(a, ctypes.c_uint16), a_row_stride, m, k,
                                  _ptr(q, ctypes.c_uint8), q_row_stride,
                                  _ptr(s, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle: invalid shape m=%d k=%d" % (m, k))
    return q, s


def _check_w8a8(qa, sa, w, sw, m, n, k, qa_row_stride):
    assert qa.dtype == np.uint8 and w.dtype == np.uint8
    assert sa.dtype == np.float32 and sw.dtype == np.float32
    assert qa.size >= (m - 1) * qa_row_stride + k and w.size >= n * k
    assert sa.size >= m * (k // K_BLOCK)
    assert sw.size >= ((n + K_BLOCK - 1) // K_BLOCK) * (k // K_BLOCK)


def gemm_w8a8(qa: np.ndarray, sa: np.ndarray, w: np.ndarray, sw: np.ndarray, m: int,
              n: int, k: int, qa_row_stride: Optional[int] = None, threads: int = 0
              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Whole W8A8 GEMM: codes ``qa`` [m, qa_row_stride] with scales ``sa``
    [m, k/128], weight codes ``w`` [n, k] with block scales ``sw``.  Returns
    (c_bits [m, n], tot [m, n], bound [m, n])."""
    qa_row_stride = k if qa_row_stride is None else int(qa_row_stride)
    qa = np.ascontiguousarray(qa, dtype=np.uint8).reshape(-1)
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    sa = np.ascontiguousarray(sa, dtype=np.float32).reshape(-1)
    sw = np.ascontiguousarray(sw, dtype=np.float32).reshape(-1)
    _check_w8a8(qa, sa, w, sw, m, n, k, qa_row_stride)
    c = np.zeros((m, n), dtype=np.uint16)
    tot = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = _load().oracle_w8a8_gemm(
        _ptr(qa, ctypes.c_uint8), qa_row_stride, _ptr(sa, ctypes.c_float),
        _ptr(w, ctypes.c_uint8), _ptr(sw, ctypes.c_float), _ptr(c, ctypes.c_uint16), n,
        m, n, k, _ptr(tot, ctypes.c_double), _ptr(bound, ctypes.c_double), int(threads))
    if rc != 0:
        raise ValueError("oracle: invalid shape m=%d n=%d k=%d" % (m, n, k))
    return c, tot, bound


def gemm_w8a8_at(qa: np.ndarray, sa: np.ndarray, w: np.ndarray, sw: np.ndarray, m: int,
                 n: int, k: int, rows: np.ndarray, cols: np.ndarray,
                 qa_row_stride: Optional[int] = None, threads: int = 0
                 ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Selected W8A8 outputs C[rows[s], cols[s]]: (c_bits, tot, bound)."""
    qa_row_stride = k if qa_row_stride is None else int(qa_row_stride)
    qa = np.ascontiguousarray(qa, dtype=np.uint8).reshape(-1)
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    sa = np.ascontiguousarray(sa, dtype=np.float32).reshape(-1)
    sw = np.ascontiguousarray(sw, dtype=np.float32).reshape(-1)
    _check_w8a8(qa, sa, w, sw, m, n, k, qa_row_stride)
    rows = np.ascontiguousarray(rows, dtype=np.uint32).reshape(-1)
    cols = np.ascontiguousarray(cols, dtype=np.uint32).reshape(-1)
    ns = rows.size
    c = np.empty(ns, dtype=np.uint16)
    tot = np.empty(ns, dtype=np.float64)
    bound = np.empty(ns, dtype=np.float64)
    rc = _load().oracle_w8a8_gemm_at(
        _ptr(qa, ctypes.c_uint8), qa_row_stride, _ptr(sa, ctypes.c_float),
        _ptr(w, ctypes.c_uint8), _ptr(sw, ctypes.c_float), m, n, k,
        _ptr(rows, ctypes.c_uint32), _ptr(cols, ctypes.c_uint32), ns,
        _ptr(c, ctypes.c_uint16), _ptr(tot, ctypes.c_double), _ptr(bound, ctypes.c_double),
        int(threads))
    if rc != 0:
        raise ValueError("oracle: invalid shape or sample index")
    return c, tot, bound


# ---------------------------------------------------------------------------
# W4A4 MX GEMV (page "w4a4_proj/mx_plan.rs", format read as OCP MXFP4: FP4
# E2M1 elements two per byte, even element in the low nibble, one E8M0 scale
# per 32 K elements of a row); the arithmetic is in w4a4_oracle.c.
# ---------------------------------------------------------------------------

MX_BLOCK = 32


def e2m1_value(code: int) -> float:
    """Value of one FP4 E2M1 code (low 4 bits)."""
    return _load().oracle_e2m1_value(int(code) & 0xF)


def e8m0_value(code: int) -> float:
    """Value of one E8M0 scale byte, 2^(code - 127) (NaN for 0xFF)."""
    return _load().oracle_e8m0_value(int(code) & 0xFF)


def gemm_w4a4(a: np.ndarray, a_scale: np.ndarray, w: np.ndarray, w_scale: np.ndarray,
              m: int, n: int, k: int, a_row_stride: Optional[int] = None,
              c_row_stride: Optional[int] = None, threads: int = 0
              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Whole W4A4 GEMM.  ``a`` packed FP4 bytes with a row pitch of
    ``a_row_stride`` elements (default k), ``a_scale`` E8M0 [m, k/32], ``w``
    packed FP4 [n, k/2], ``w_scale`` E8M0 [n, k/32].  Returns (c_bits [m,
    c_row_stride], tot [m, n], bound [m, n])."""
    a_row_stride = k if a_row_stride is None else int(a_row_stride)
    c_row_stride = n if c_row_stride is None else int(c_row_stride)
    a = np.ascontiguousarray(a, dtype=np.uint8).reshape(-1)
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.uint8).reshape(-1)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.uint8).reshape(-1)
    assert a.size >= (m - 1) * (a_row_stride // 2) + k // 2 and w.size >= n * k // 2
    assert a_scale.size >= m * (k // MX_BLOCK) and w_scale.size >= n * (k // MX_BLOCK)
    c = np.zeros((m, c_row_stride), dtype=np.uint16)
    tot = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = _load().oracle_w4a4_gemm(
        _ptr(a, ctypes.c_uint8), a_row_stride, _ptr(a_scale, ctypes.c_uint8),
        _ptr(w, ctypes.c_uint8), _ptr(w_scale, ctypes.c_uint8), _ptr(c, ctypes.c_uint16),
        c_row_stride, m, n, k, _ptr(tot, ctypes.c_double), _ptr(bound, ctypes.c_double),
        int(threads))
    if rc != 0:
        raise ValueError("oracle: invalid W4A4 shape m=%d n=%d k=%d" % (m, n, k))
    return c, tot, bound


def gemm_w4a4_at(a: np.ndarray, a_scale: np.ndarray, w: np.ndarray, w_scale: np.ndarray,
                 m: int, n: int, k: int, rows: np.ndarray, cols: np.ndarray,
                 a_row_stride: Optional[int] = None, threads: int = 0
                 ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Selected W4A4 outputs C[rows[s], cols[s]] (operands as for
    gemm_w4a4): (c_bits uint16 [s], tot float64 [s], bound float64 [s])."""
    a_row_stride = k if a_row_stride is None else int(a_row_stride)
    a = np.ascontiguousarray(a, dtype=np.uint8).reshape(-1)
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.uint8).reshape(-1)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.uint8).reshape(-1)
    assert a.size >= (m - 1) * (a_row_stride // 2) + k // 2 and w.size >= n * k // 2
    assert a_scale.size >= m * (k // MX_BLOCK) and w_scale.size >= n * (k // MX_BLOCK)
    rows = np.ascontiguousarray(rows, dtype=np.uint32).reshape(-1)
    cols = np.ascontiguousarray(cols, dtype=np.uint32).reshape(-1)
    ns = rows.size
    c = np.zeros(ns, dtype=np.uint16)
    tot = np.empty(ns, dtype=np.float64)
    bound = np.empty(ns, dtype=np.float64)
    rc = _load().oracle_w4a4_gemm_at(
        _ptr(a, ctypes.c_uint8), a_row_stride, _ptr(a_scale, ctypes.c_uint8),
        _ptr(w, ctypes.c_uint8), _ptr(w_scale, ctypes.c_uint8), m, n, k,
        _ptr(rows, ctypes.c_uint32), _ptr(cols, ctypes.c_uint32), ns, _ptr(c, ctypes.c_uint16),
        _ptr(tot, ctypes.c_double), _ptr(bound, ctypes.c_double), int(threads))
    if rc != 0:
        raise ValueError("oracle: invalid W4A4 shape or sample index")
    return c, tot, bound


# ---------------------------------------------------------------------------
# Parity tolerance.  A GPU result g for one output passes iff, in double,
#     |g - oracle| <= 2^-8 * B + ulp(oracle)
# where B = sum |a*w*s| over the output's K range and ulp(v) is the BF16
# spacing at v: 2^(max(floor(log2|v|), -126) - 7), with ulp(0) = 2^-133.
# A NaN or infinite GPU value fails.
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact BF16 bits -> float64 (vectorised form of bf16_value)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """BF16 spacing at each value: 2^(max(floor(log2|v|), -126) - 7), 2^-133
    at zero, NaN where v is not finite."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    fin = np.isfinite(v)
    v = np.where(fin, v, 1.0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.where(v > 0, np.maximum(e, -126.0), -126.0)
    return np.where(fin, np.ldexp(1.0, (e - 7).astype(np.int64)), np.nan)


def within_tolerance(gpu_bits: np.ndarray, oracle_bits: np.ndarray,
                     bound: np.ndarray) -> np.ndarray:
    """Boolean mask: True where the GPU output passes the parity bar."""
    g = bf16_bits_to_f64(gpu_bits)
    o = bf16_bits_to_f64(oracle_bits)
    lim = np.ldexp(np.asarray(bound, dtype=np.float64), -8) + bf16_ulp(o)
    with np.errstate(invalid="ignore"):
        ok = np.isfinite(g) & (np.abs(g - o) <= lim)
    return ok
