"""Seeded synthetic inputs for the block-scaled FP8 W8A16 GEMM.

This module only *makes operands*: BF16 activations, E4M3 weight codes with
their FP32 per-128x128-block scales, and padded buffers.  It holds none of
the GEMM's arithmetic (no decode, no dot products, no output rounding) and
imports neither the oracle nor the product package, so both sides can take
the same inputs from it.

Recipe (the five workloads of the W8A16 small-M projection GEMM):

* A: float32 draws from N(0, 1) (numpy ``default_rng(seed)``, drawn first),
  rounded to BF16 by torch's float32 -> bfloat16 cast (round to nearest
  even).  Row pitch ``a_row_stride``; pad columns hold the BF16 NaN 0x7FC0
  so that reading them would poison the result.
* W: float32 draws from N(0, 0.02) (drawn second, standard deviation 0.02),
  quantized per 128x128 block: scale s = amax/448 in float32, codes =
  float8_e4m3fn(clamp(w / s, -448, 448)) by torch's cast (round to nearest
  even).  An all-zero block gets s = 0 and codes 0x00.  A ragged last N
  block is quantized over the rows it has.
* ``zero_every``: block (nb, kb) is forced to all-zero codes when
  (nb * (K/128) + kb) % zero_every == 0; its scale is left as drawn.
* ``log_scales``: after quantizing, every scale is replaced by 2^u with u
  drawn from U(lo, hi) in float64 (drawn third) and rounded to float32.
* C: a buffer of ``c_row_stride`` columns (and optional extra rows) filled
  with the sentinel 0xFFFF, which a correct GEMM leaves alone outside
  [m, n].
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

K_BLOCK = 128
E4M3_MAX = 448.0
A_PAD_BITS = 0x7FC0   # BF16 quiet NaN
C_SENTINEL = 0xFFFF


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    m: int
    n: int
    k: int
    a_row_stride: int
    c_row_stride: int
    seed: int
    zero_every: int = 0
    log_scales: Optional[Tuple[float, float]] = None
    c_extra_rows: int = 0

    @property
    def scale_shape(self) -> Tuple[int, int]:
        return ((self.n + K_BLOCK - 1) // K_BLOCK, self.k // K_BLOCK)

    def algorithmic_bytes(self) -> int:
        """Bytes the operation must move at least once: the weight codes,
        the scales, the used part of A and the written part of C
        (N*K + 4*(N/128)*(K/128) + 2*M*K + 2*M*N)."""
        nb, kb = self.scale_shape
        return (self.n * self.k + 4 * nb * kb + 2 * self.m * self.k
                + 2 * self.m * self.n)

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


WORKLOADS = (
    Workload("m1_n256_k256", 1, 256, 256, 256, 256, 1001),
    Workload("m8_n4096_k4096", 8, 4096, 4096, 4096, 4096, 1002),
    Workload("m16_n12288_k5120", 16, 12288, 5120, 5120, 12288, 1003),
    Workload("m32_n6144_k2048_strided", 32, 6144, 2048, 2560, 8192, 1004,
             c_extra_rows=2),
    Workload("m128_n8192_k8192", 128, 8192, 8192, 8192, 8192, 1005,
             zero_every=8, log_scales=(-12.0, -4.0)),
)


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for wl in WORKLOADS:
        if wl.name == name_or_index:
            return wl
    raise KeyError(name_or_index)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits (uint16) with torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 (already inside [-448, 448]) -> OCP E4M3FN bytes with torch's
    round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_blockwise(wf: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-128x128-block E4M3 quantization with scale = amax/448 (float32).
    ``wf`` is float32 [n, k] with k % 128 == 0.  Returns (codes uint8 [n, k],
    scales float32 [ceil(n/128), k/128])."""
    n, k = wf.shape
    assert k % K_BLOCK == 0
    nb, kb = (n + K_BLOCK - 1) // K_BLOCK, k // K_BLOCK
    pad = nb * K_BLOCK - n
    wp = np.pad(wf, ((0, pad), (0, 0))) if pad else wf
    blocks = wp.reshape(nb, K_BLOCK, kb, K_BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = blocks / safe[:, None, :, None]
    q = np.clip(q, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = to_e4m3_codes(q.reshape(nb * K_BLOCK, k))[:n]
    codes = np.where(np.repeat(np.repeat(scale == 0, K_BLOCK, 0), K_BLOCK, 1)[:n],
                     np.uint8(0), codes).astype(np.uint8)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scale)


@dataclasses.dataclass
class Problem:
    """Host operands of one GEMM call.  ``a`` is [m, a_row_stride] BF16 bits,
    ``w`` [n, k] E4M3 codes, ``scale`` [ceil(n/128), k/128] float32, ``c``
    the initial output buffer [m + c_extra_rows, c_row_stride] BF16 bits."""
    m: int
    n: int
    k: int
    a_row_stride: int
    c_row_stride: int
    a: np.ndarray
    w: np.ndarray
    scale: np.ndarray
    c: np.ndarray
    seed: int


def make_problem(m: int, n: int, k: int, seed: int,
                 a_row_stride: Optional[int] = None,
                 c_row_stride: Optional[int] = None,
                 w_std: float = 0.02, zero_every: int = 0,
                 log_scales: Optional[Tuple[float, float]] = None,
                 c_extra_rows: int = 0) -> Problem:
    a_row_stride = k if a_row_stride is None else a_row_stride
    c_row_stride = n if c_row_stride is None else c_row_stride
    rng = np.random.default_rng(seed)
    af = rng.standard_normal((m, k), dtype=np.float32)
    a = np.full((m, a_row_stride), A_PAD_BITS, dtype=np.uint16)
    a[:, :k] = to_bf16_bits(af)
    del af
    wf = rng.standard_normal((n, k), dtype=np.float32) * np.float32(w_std)
    codes, scale = quantize_blockwise(wf)
    del wf
    kb = k // K_BLOCK
    if zero_every:
        nb = scale.shape[0]
        ids = np.arange(nb)[:, None] * kb + np.arange(kb)[None, :]
        zero = (ids % zero_every) == 0
        zmask = np.repeat(np.repeat(zero, K_BLOCK, 0), K_BLOCK, 1)[:n]
        codes[zmask] = 0
    if log_scales is not None:
        lo, hi = log_scales
        u = rng.uniform(lo, hi, size=scale.shape)
        scale = np.exp2(u).astype(np.float32)
    c = np.full((m + c_extra_rows, c_row_stride), C_SENTINEL, dtype=np.uint16)
    return Problem(m, n, k, a_row_stride, c_row_stride, a, codes, scale, c,
                   seed)


def make_workload(wl: Workload) -> Problem:
    return make_problem(wl.m, wl.n, wl.k, wl.seed, wl.a_row_stride,
                        wl.c_row_stride, zero_every=wl.zero_every,
                        log_scales=wl.log_scales,
                        c_extra_rows=wl.c_extra_rows)


def sample_indices(m: int, n: int, count: int, seed: int
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Output positions to check at full size: every row's first and last
    column, every 128-column block edge of row 0 and m-1, plus uniform
    random picks."""
    rng = np.random.default_rng(seed)
    rows = [np.arange(m), np.arange(m)]
    cols = [np.zeros(m, np.int64), np.full(m, n - 1)]
    edges = np.unique(np.concatenate([np.arange(0, n, K_BLOCK),
                                      np.arange(K_BLOCK - 1, n, K_BLOCK)]))
    for r in {0, m - 1}:
        rows.append(np.full(edges.size, r))
        cols.append(edges)
    rows.append(rng.integers(0, m, count))
    cols.append(rng.integers(0, n, count))
    return (np.concatenate(rows).astype(np.uint32),
            np.concatenate(cols).astype(np.uint32))


# ---------------------------------------------------------------------------
# W4A4 MX operands (page "w4a4_proj/mx_plan.rs" plans the projection; the
# format read as OCP MXFP4): FP4 E2M1 elements, two per byte with the even
# element in the low nibble, one E8M0 scale byte per 32 consecutive K
# elements of a row.
#
# Recipe: A float32 N(0, 1) [m, k] (drawn first), W float32 N(0, 0.02)
# [n, k] (drawn second), each quantized per 32-element block as the MX
# format's conversion does: shared exponent e = floor(log2(amax)) - 2 (2 is
# E2M1's largest exponent), clamped to [-127, 127], scale byte e + 127;
# elements = E2M1 round-to-nearest-even of v / 2^e, saturated to +-6; an
# all-zero block gets scale byte 0 (2^-127) and zero elements.  A's row
# pitch is in elements (even); pad bytes hold 0x77 (6.0 in both nibbles),
# which would change the result if read.
# ---------------------------------------------------------------------------

MX_BLOCK = 32
A_PAD_FP4 = 0x77

# E2M1 magnitude code boundaries for round-to-nearest-even: |x| in
# (lo, hi) goes to the code; a tie goes to the even code.
_E2M1_MAGS = np.float32([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def to_e2m1_codes(x: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (uint8, 0..15) nearest to float32 ``x``, ties to the
    even code, saturating to +-6."""
    x = np.asarray(x, dtype=np.float32)
    mag = np.abs(x)
    d = np.abs(mag[..., None] - _E2M1_MAGS)            # distances to the 8 magnitudes
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equidistant codes take the even one (ties occur between a pair)
    even = cand & ((np.arange(8) % 2) == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    code = np.where(mag > 6.0, 7, code).astype(np.uint8)
    return (code | np.where(np.signbit(x), np.uint8(8), np.uint8(0))).astype(np.uint8)


def quantize_mx(xf: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantization of float32 [r, k] (k % 32 == 0): returns (packed
    codes uint8 [r, k/2], scale bytes uint8 [r, k/32])."""
    r, k = xf.shape
    assert k % MX_BLOCK == 0
    blocks = xf.reshape(r, k // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0
    e = np.clip(np.where(amax > 0, e, -127.0), -127.0, 127.0)
    scaled = (blocks / np.exp2(e)[..., None].astype(np.float32)).astype(np.float32)
    codes = to_e2m1_codes(scaled).reshape(r, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray((e + 127).astype(np.uint8))


@dataclasses.dataclass
class MxProblem:
    """Host operands of one W4A4 call: ``a`` [m, a_row_stride / 2] packed
    FP4 bytes, ``a_scale`` [m, k/32], ``w`` [n, k/2], ``w_scale`` [n, k/32]
    (E8M0 bytes), ``c`` [m + c_extra_rows, c_row_stride] BF16 bits."""
    m: int
    n: int
    k: int
    a_row_stride: int
    c_row_stride: int
    a: np.ndarray
    a_scale: np.ndarray
    w: np.ndarray
    w_scale: np.ndarray
    c: np.ndarray
    seed: int

    def algorithmic_bytes(self) -> int:
        """FP4 weight and activations once, their scales once, C once."""
        return (self.n * self.k // 2 + self.n * self.k // MX_BLOCK + self.m * self.k // 2 +
                self.m * self.k // MX_BLOCK + 2 * self.m * self.n)


def make_mx_problem(m: int, n: int, k: int, seed: int, a_row_stride: Optional[int] = None,
                    c_row_stride: Optional[int] = None, w_std: float = 0.02,
                    c_extra_rows: int = 0) -> MxProblem:
    a_row_stride = k if a_row_stride is None else a_row_stride
    c_row_stride = n if c_row_stride is None else c_row_stride
    assert a_row_stride % 2 == 0 and a_row_stride >= k
    rng = np.random.default_rng(seed)
    af = rng.standard_normal((m, k), dtype=np.float32)
    apk, asc = quantize_mx(af)
    a = np.full((m, a_row_stride // 2), A_PAD_FP4, dtype=np.uint8)
    a[:, :k // 2] = apk
    wf = rng.standard_normal((n, k), dtype=np.float32) * np.float32(w_std)
    w, wsc = quantize_mx(wf)
    c = np.full((m + c_extra_rows, c_row_stride), C_SENTINEL, dtype=np.uint16)
    return MxProblem(m, n, k, a_row_stride, c_row_stride, a, asc, w, wsc, c, seed)
