"""Block-scaled FP8 W8A16 small-M GEMM for MI355X (gfx950).

Thin binding over ``libw8a16.so`` (the C ABI in ``include/w8a16.h``):
argument marshalling only.  Every step of the GEMM runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream.  If the
library has not been built, every call raises -- there is no fallback.

    C[i, j] = bf16( sum_b S[j//128, b] * sum_t A[i, 128b+t] * W[j, 128b+t] )

A is BF16 [m, k] (any row pitch that is a multiple of 8), W is FP8 E4M3
[n, k] (torch.float8_e4m3fn or its uint8 bytes), S is float32
[ceil(n/128), k/128], C is BF16 [m, n] (any row pitch >= n).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8a16.so")

OK = 0
ERR_M_ZERO = 1
ERR_K_NOT_MULT_128 = 2
ERR_PITCH_TOO_SHORT = 3
ERR_A_STRIDE_ALIGN = 4
ERR_N_ZERO = 5
ERR_NULL_PTR = 6
ERR_BAD_PLAN = 7
ERR_HIP = 8
ERR_WORKSPACE = 9
ERR_ENV = 10

KERNEL_STREAM = 1
KERNEL_TILE = 2
KERNEL_RING = 3
KERNEL_W8A8 = 4
KERNEL_W4A4 = 5
KERNEL_W4A4_PS = 6

FLAG_DIRECT = 1
FLAG_A8 = 2
FLAG_XCD_LOCAL = 4

# Symbols the C ABI exports (include/w8a16.h).
EXPORTS = ("w8a16_check_args", "w8a16_plan", "w8a16_plan_finalize", "w8a16_gemm",
           "w8a16_gemm_planned", "w8a16_gemm_noalloc", "w8a16_plan_batched", "w8a16_gemm_batched",
           "w8a16_act_quant_fp8", "w8a16_plan_w8a8", "w8a16_gemm_w8a8",
           "w8a16_gemm_w8a8_planned", "w8a16_gemm_w4a4", "w8a16_plan_w4a4",
           "w8a16_gemm_w4a4_planned", "w8a16_status_string", "w8a16_last_error")

MAX_BATCH = 8


class W8A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("w8a16 status %d: %s" % (status, message))
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_uint32), ("m_blocks", ctypes.c_uint32),
                ("n_blocks", ctypes.c_uint32), ("splits", ctypes.c_uint32),
                ("steps_per_split", ctypes.c_uint32), ("m_tiles", ctypes.c_uint32),
                ("n_tiles", ctypes.c_uint32), ("grid", ctypes.c_uint32),
                ("block", ctypes.c_uint32), ("lds_bytes", ctypes.c_uint32),
                ("workspace_bytes", ctypes.c_uint64),
                ("counter_count", ctypes.c_uint32), ("cu_count", ctypes.c_uint32),
                ("depth", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("waves", ctypes.c_uint32), ("stage_steps", ctypes.c_uint32),
                ("a_depth", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class GemmDesc(ctypes.Structure):
    """One GEMM of a batched call (w8a16_gemm_desc_t): device addresses and
    the w8a16_gemm() scalars."""
    _fields_ = [("a", ctypes.c_void_p), ("w_fp8", ctypes.c_void_p),
                ("block_scale", ctypes.c_void_p), ("c", ctypes.c_void_p),
                ("a_row_stride", ctypes.c_uint32), ("c_row_stride", ctypes.c_uint32),
                ("m", ctypes.c_uint32), ("n", ctypes.c_uint32), ("k", ctypes.c_uint32)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libw8a16.so (raises if it is missing: build it first with
    ``python -m block_scaled_fp8_w8a16_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libw8a16.so is not built (%s); run "
                              "python -m block_scaled_fp8_w8a16_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        u32, vp = ctypes.c_uint32, ctypes.c_void_p
        lib.w8a16_check_args.argtypes = [u32] * 5
        lib.w8a16_check_args.restype = ctypes.c_int
        lib.w8a16_plan.argtypes = [u32, u32, u32, u32, ctypes.POINTER(Plan)]
        lib.w8a16_plan.restype = ctypes.c_int
        lib.w8a16_plan_finalize.argtypes = [u32, u32, u32, ctypes.POINTER(Plan)]
        lib.w8a16_plan_finalize.restype = ctypes.c_int
        lib.w8a16_gemm.argtypes = [vp, u32, vp, vp, vp, u32, u32, u32, u32, vp]
        lib.w8a16_gemm.restype = ctypes.c_int
        lib.w8a16_gemm_planned.argtypes = [vp, u32, vp, vp, vp, u32, u32, u32, u32,
                                           ctypes.POINTER(Plan), vp]
        lib.w8a16_gemm_planned.restype = ctypes.c_int
        lib.w8a16_gemm_noalloc.argtypes = [vp, u32, vp, vp, vp, u32, u32, u32, u32, vp]
        lib.w8a16_gemm_noalloc.restype = ctypes.c_int
        lib.w8a16_plan_batched.argtypes = [ctypes.POINTER(GemmDesc), u32, u32,
                                           ctypes.POINTER(Plan)]
        lib.w8a16_plan_batched.restype = ctypes.c_int
        lib.w8a16_gemm_batched.argtypes = [ctypes.POINTER(GemmDesc), u32, vp]
        lib.w8a16_gemm_batched.restype = ctypes.c_int
        lib.w8a16_act_quant_fp8.argtypes = [vp, u32, vp, u32, vp, u32, u32, vp]
        lib.w8a16_act_quant_fp8.restype = ctypes.c_int
        lib.w8a16_plan_w8a8.argtypes = [u32, u32, u32, u32, ctypes.POINTER(Plan)]
        lib.w8a16_plan_w8a8.restype = ctypes.c_int
        lib.w8a16_gemm_w8a8.argtypes = [vp, u32, vp, vp, vp, vp, u32, u32, u32, u32, vp]
        lib.w8a16_gemm_w8a8.restype = ctypes.c_int
        lib.w8a16_gemm_w8a8_planned.argtypes = [vp, u32, vp, vp, vp, vp, u32, u32, u32, u32,
                                                ctypes.POINTER(Plan), vp]
        lib.w8a16_gemm_w8a8_planned.restype = ctypes.c_int
        lib.w8a16_gemm_w4a4.argtypes = [vp, u32, vp, vp, vp, vp, u32, u32, u32, u32, vp]
        lib.w8a16_gemm_w4a4.restype = ctypes.c_int
        lib.w8a16_plan_w4a4.argtypes = [u32, u32, u32, u32, ctypes.POINTER(Plan)]
        lib.w8a16_plan_w4a4.restype = ctypes.c_int
        lib.w8a16_gemm_w4a4_planned.argtypes = [vp, u32, vp, vp, vp, vp, u32, u32, u32, u32,
                                                ctypes.POINTER(Plan), vp]
        lib.w8a16_gemm_w4a4_planned.restype = ctypes.c_int
        lib.w8a16_status_string.argtypes = [ctypes.c_int]
        lib.w8a16_status_string.restype = ctypes.c_char_p
        lib.w8a16_last_error.argtypes = []
        lib.w8a16_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def last_error() -> str:
    return library().w8a16_last_error().decode()


def status_string(status: int) -> str:
    return library().w8a16_status_string(int(status)).decode()


def _raise_if(status: int):
    if status != OK:
        raise W8A16Error(status, last_error() or status_string(status))


def check_args(m: int, n: int, k: int, a_row_stride: int, c_row_stride: int) -> int:
    """Status of the scalar argument checks (no GPU call)."""
    return int(library().w8a16_check_args(m, n, k, a_row_stride, c_row_stride))


def plan(m: int, n: int, k: int, cu_count: int = 0) -> Plan:
    """Default launch plan (no GPU call)."""
    p = Plan()
    _raise_if(library().w8a16_plan(m, n, k, cu_count, ctypes.byref(p)))
    return p


def make_plan(m: int, n: int, k: int, kernel: int, m_blocks: int, n_blocks: int,
              splits: int, depth: int = 2, flags: int = 0, waves: int = 4,
              cu_count: int = 0, stage_steps: int = 0, a_depth: int = 0) -> Plan:
    """A caller-chosen plan, checked and completed by the library."""
    p = Plan()
    p.kernel, p.m_blocks, p.n_blocks, p.splits, p.cu_count = \
        kernel, m_blocks, n_blocks, splits, cu_count
    p.depth, p.flags, p.waves = depth, flags, waves
    p.stage_steps, p.a_depth = stage_steps, a_depth
    _raise_if(library().w8a16_plan_finalize(m, n, k, ctypes.byref(p)))
    return p


def gemm_raw(a_ptr: int, a_row_stride: int, w_ptr: int, scale_ptr: int, c_ptr: int,
             c_row_stride: int, m: int, n: int, k: int, stream: int = 0,
             plan_: Optional[Plan] = None) -> int:
    """Direct call of the C ABI with device addresses; returns the status."""
    lib = library()
    if plan_ is None:
        return int(lib.w8a16_gemm(a_ptr, a_row_stride, w_ptr, scale_ptr, c_ptr,
                                  c_row_stride, m, n, k, stream))
    return int(lib.w8a16_gemm_planned(a_ptr, a_row_stride, w_ptr, scale_ptr, c_ptr,
                                      c_row_stride, m, n, k, ctypes.byref(plan_),
                                      stream))


def gemm_noalloc_raw(a_ptr: int, a_row_stride: int, w_ptr: int, scale_ptr: int, c_ptr: int,
                     c_row_stride: int, m: int, n: int, k: int, stream: int = 0) -> int:
    """w8a16_gemm_noalloc with device addresses (split-K scratch from the
    library's static device array, no allocation); returns the status."""
    return int(library().w8a16_gemm_noalloc(a_ptr, a_row_stride, w_ptr, scale_ptr, c_ptr,
                                            c_row_stride, m, n, k, stream))


NOALLOC_WORKSPACE_BYTES = 16 << 20
NOALLOC_COUNTERS = 1 << 18


def gemm(a, w, scale, c=None, *, plan_: Optional[Plan] = None, stream=None):
    """C = A @ dequant(W)^T on the current (or given) torch stream.

    a: bfloat16 [m, k] CUDA tensor, unit column stride, row stride a multiple
    of 8.  w: float8_e4m3fn or uint8 [n, k] contiguous.  scale: float32
    [ceil(n/128), k/128] contiguous.  c: optional bfloat16 [m, n] output with
    unit column stride (a new contiguous tensor if None).  Returns c."""
    import torch
    if a.dim() != 2 or w.dim() != 2:
        raise ValueError("a and w must be 2-D")
    m, k = a.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("w must be [n, k] with the k of a")
    if a.dtype != torch.bfloat16 or a.stride(1) != 1:
        raise ValueError("a must be bfloat16 with unit column stride")
    if w.dtype not in (torch.uint8, torch.float8_e4m3fn) or not w.is_contiguous():
        raise ValueError("w must be contiguous float8_e4m3fn or uint8")
    if scale.dtype != torch.float32 or not scale.is_contiguous():
        raise ValueError("scale must be contiguous float32")
    nb = (n + 127) // 128
    if scale.numel() < nb * (k // 128 if k % 128 == 0 else 0):
        raise ValueError("scale must hold [ceil(n/128), k/128] values")
    if c is None:
        c = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if c.dtype != torch.bfloat16 or c.stride(1) != 1 or tuple(c.shape) != (m, n):
        raise ValueError("c must be bfloat16 [m, n] with unit column stride")
    for t in (a, w, scale, c):
        if not t.is_cuda:
            raise ValueError("all operands must be GPU tensors")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    a_rs = a.stride(0) if m > 1 else max(a.stride(0), k)
    c_rs = c.stride(0) if m > 1 else max(c.stride(0), n)
    st = gemm_raw(a.data_ptr(), a_rs, w.data_ptr(), scale.data_ptr(), c.data_ptr(),
                  c_rs, m, n, k, stream.cuda_stream, plan_)
    _raise_if(st)
    return c


def _desc_array(descs):
    arr = (GemmDesc * max(1, len(descs)))()
    for i, d in enumerate(descs):
        arr[i] = d if isinstance(d, GemmDesc) else GemmDesc(**d)
    return arr


def plan_batched(shapes, cu_count: int = 0) -> Plan:
    """Plan of a batched call for [(m, n, k), ...] (no GPU call)."""
    descs = [GemmDesc(m=m, n=n, k=k) for (m, n, k) in shapes]
    p = Plan()
    _raise_if(library().w8a16_plan_batched(_desc_array(descs), len(descs), cu_count,
                                           ctypes.byref(p)))
    return p


def gemm_batched_raw(descs, stream: int = 0) -> int:
    """Direct call of w8a16_gemm_batched with GemmDesc (or dict) entries;
    returns the status."""
    return int(library().w8a16_gemm_batched(_desc_array(descs), len(descs), stream))


def gemm_batched(problems, *, stream=None):
    """Several independent GEMMs in one launch.  problems: a list of
    (a, w, scale, c) tuples of CUDA tensors laid out as for gemm() (c is
    required here).  Returns the list of c tensors."""
    import torch
    descs = []
    for a, w, scale, c in problems:
        if a.dim() != 2 or w.dim() != 2 or c.dim() != 2:
            raise ValueError("a, w and c must be 2-D")
        m, k = a.shape
        n = w.shape[0]
        if w.shape[1] != k or tuple(c.shape) != (m, n):
            raise ValueError("shapes must be a [m, k], w [n, k], c [m, n]")
        if a.dtype != torch.bfloat16 or a.stride(1) != 1:
            raise ValueError("a must be bfloat16 with unit column stride")
        if w.dtype not in (torch.uint8, torch.float8_e4m3fn) or not w.is_contiguous():
            raise ValueError("w must be contiguous float8_e4m3fn or uint8")
        if scale.dtype != torch.float32 or not scale.is_contiguous():
            raise ValueError("scale must be contiguous float32")
        if c.dtype != torch.bfloat16 or c.stride(1) != 1:
            raise ValueError("c must be bfloat16 with unit column stride")
        for t in (a, w, scale, c):
            if not t.is_cuda:
                raise ValueError("all operands must be GPU tensors")
        descs.append(GemmDesc(a=a.data_ptr(), w_fp8=w.data_ptr(), block_scale=scale.data_ptr(),
                              c=c.data_ptr(),
                              a_row_stride=a.stride(0) if m > 1 else max(a.stride(0), k),
                              c_row_stride=c.stride(0) if m > 1 else max(c.stride(0), n),
                              m=m, n=n, k=k))
    if stream is None:
        stream = torch.cuda.current_stream(problems[0][0].device)
    _raise_if(gemm_batched_raw(descs, stream.cuda_stream))
    return [p[3] for p in problems]


# ------------------------------------------------- FP8 activations, W8A8

def plan_w8a8(m: int, n: int, k: int, cu_count: int = 0) -> Plan:
    """Default plan of the W8A8 GEMM (no GPU call)."""
    p = Plan()
    _raise_if(library().w8a16_plan_w8a8(m, n, k, cu_count, ctypes.byref(p)))
    return p


def act_quant_fp8_raw(a_ptr: int, a_row_stride: int, q_ptr: int, q_row_stride: int,
                      scales_ptr: int, m: int, k: int, stream: int = 0) -> int:
    """Direct call of w8a16_act_quant_fp8; returns the status."""
    return int(library().w8a16_act_quant_fp8(a_ptr, a_row_stride, q_ptr, q_row_stride,
                                             scales_ptr, m, k, stream))


def gemm_w8a8_raw(qa_ptr: int, qa_row_stride: int, a_scales_ptr: int, w_ptr: int,
                  scale_ptr: int, c_ptr: int, c_row_stride: int, m: int, n: int, k: int,
                  stream: int = 0, plan_: Optional[Plan] = None) -> int:
    """Direct call of w8a16_gemm_w8a8 (or its planned form); returns the status."""
    lib = library()
    if plan_ is None:
        return int(lib.w8a16_gemm_w8a8(qa_ptr, qa_row_stride, a_scales_ptr, w_ptr, scale_ptr,
                                       c_ptr, c_row_stride, m, n, k, stream))
    return int(lib.w8a16_gemm_w8a8_planned(qa_ptr, qa_row_stride, a_scales_ptr, w_ptr,
                                           scale_ptr, c_ptr, c_row_stride, m, n, k,
                                           ctypes.byref(plan_), stream))


def plan_w4a4(m: int, n: int, k: int, cu_count: int = 0) -> Plan:
    """Default plan of the W4A4 MX GEMV (no GPU call)."""
    p = Plan()
    _raise_if(library().w8a16_plan_w4a4(m, n, k, cu_count, ctypes.byref(p)))
    return p


def gemm_w4a4_raw(a_ptr: int, a_row_stride: int, a_scale_ptr: int, w_ptr: int,
                  w_scale_ptr: int, c_ptr: int, c_row_stride: int, m: int, n: int, k: int,
                  stream: int = 0, plan_: Optional[Plan] = None) -> int:
    """Direct call of w8a16_gemm_w4a4 (or its planned form) with device
    addresses; a_row_stride in FP4 elements.  Returns the status."""
    lib = library()
    if plan_ is None:
        return int(lib.w8a16_gemm_w4a4(a_ptr, a_row_stride, a_scale_ptr, w_ptr, w_scale_ptr,
                                       c_ptr, c_row_stride, m, n, k, stream))
    return int(lib.w8a16_gemm_w4a4_planned(a_ptr, a_row_stride, a_scale_ptr, w_ptr,
                                           w_scale_ptr, c_ptr, c_row_stride, m, n, k,
                                           ctypes.byref(plan_), stream))


def gemm_w4a4(a, a_scale, w, w_scale, k: int, c=None, *, plan_: Optional[Plan] = None,
              stream=None):
    """W4A4 MX GEMV on the current (or given) torch stream.

    a: uint8 [m, >= k/2] packed FP4 (two E2M1 per byte, even element in the
    low nibble), unit column stride, row stride a multiple of 16 bytes;
    a_scale: uint8 [m, k/32] E8M0, contiguous; w: uint8 [n, k/2] packed FP4,
    contiguous; w_scale: uint8 [n, k/32] E8M0, contiguous.  c: optional
    bfloat16 [m, n] output with unit column stride.  Returns c."""
    import torch
    m, n = a.shape[0], w.shape[0]
    for name, t in (("a", a), ("a_scale", a_scale), ("w", w), ("w_scale", w_scale)):
        if t.dtype != torch.uint8:
            raise ValueError("%s must be uint8 (packed FP4 or E8M0 bytes)" % name)
    if a.stride(1) != 1 or not (w.is_contiguous() and a_scale.is_contiguous() and
                                w_scale.is_contiguous()):
        raise ValueError("a needs unit column stride; w and the scales must be contiguous")
    if w.shape[1] != k // 2 or a.shape[1] < k // 2:
        raise ValueError("w must be [n, k/2] bytes and a at least k/2 bytes wide")
    if a_scale.shape != (m, k // 32) or w_scale.shape != (n, k // 32):
        raise ValueError("scales must be [rows, k/32]")
    if not (a.is_cuda and a_scale.is_cuda and w.is_cuda and w_scale.is_cuda):
        raise ValueError("operands must be CUDA tensors")
    if c is None:
        c = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    elif c.dtype != torch.bfloat16 or c.stride(1) != 1 or tuple(c.shape) != (m, n):
        raise ValueError("c must be bfloat16 [m, n] with unit column stride")
    stream = torch.cuda.current_stream() if stream is None else stream
    st = gemm_w4a4_raw(a.data_ptr(), a.stride(0) * 2, a_scale.data_ptr(), w.data_ptr(),
                       w_scale.data_ptr(), c.data_ptr(), c.stride(0), m, n, k,
                       stream.cuda_stream, plan_)
    _raise_if(st)
    return c


def act_quant_fp8(a, *, stream=None):
    """Per-token, per-128-group FP8 quantization of a bfloat16 [m, k] CUDA
    tensor (unit column stride, row stride a multiple of 8).  Returns
    (codes uint8 [m, k], scales float32 [m, k/128])."""
    import torch
    if a.dim() != 2 or a.dtype != torch.bfloat16 or a.stride(1) != 1 or not a.is_cuda:
        raise ValueError("a must be a 2-D bfloat16 CUDA tensor with unit column stride")
    m, k = a.shape
    q = torch.empty((m, k), dtype=torch.uint8, device=a.device)
    s = torch.empty((m, max(0, k // 128)), dtype=torch.float32, device=a.device)
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    a_rs = a.stride(0) if m > 1 else max(a.stride(0), k)
    _raise_if(act_quant_fp8_raw(a.data_ptr(), a_rs, q.data_ptr(), k,
                                s.data_ptr(), m, k, stream.cuda_stream))
    return q, s


def gemm_w8a8(qa, a_scales, w, scale, c=None, *, plan_: Optional[Plan] = None, stream=None):
    """C = (FP8 activations qa [m, k] with scales [m, k/128]) @ dequant(W)^T
    on the current (or given) torch stream.  Returns c (bfloat16 [m, n])."""
    import torch
    if qa.dim() != 2 or w.dim() != 2:
        raise ValueError("qa and w must be 2-D")
    m, k = qa.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("w must be [n, k] with the k of qa")
    for t in (qa, w):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or t.stride(1) != 1:
            raise ValueError("qa and w must be float8_e4m3fn or uint8 with unit column stride")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    for t in (a_scales, scale):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("scales must be contiguous float32")
    ks = k // 128 if k % 128 == 0 else 0
    if a_scales.numel() < m * ks or scale.numel() < (n + 127) // 128 * ks:
        raise ValueError("a_scales must hold [m, k/128] and scale [ceil(n/128), k/128] values")
    if c is None:
        c = torch.empty((m, n), dtype=torch.bfloat16, device=qa.device)
    if c.dtype != torch.bfloat16 or c.stride(1) != 1 or tuple(c.shape) != (m, n):
        raise ValueError("c must be bfloat16 [m, n] with unit column stride")
    for t in (qa, a_scales, w, scale, c):
        if not t.is_cuda:
            raise ValueError("all operands must be GPU tensors")
    if stream is None:
        stream = torch.cuda.current_stream(qa.device)
    q_rs = qa.stride(0) if m > 1 else max(qa.stride(0), k)
    c_rs = c.stride(0) if m > 1 else max(c.stride(0), n)
    _raise_if(gemm_w8a8_raw(qa.data_ptr(), q_rs, a_scales.data_ptr(), w.data_ptr(),
                            scale.data_ptr(), c.data_ptr(), c_rs, m, n, k, stream.cuda_stream,
                            plan_))
    return c
