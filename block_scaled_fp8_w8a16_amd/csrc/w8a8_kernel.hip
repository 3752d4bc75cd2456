// FP8 activation quantizer and the block-scaled W8A8 GEMM it feeds (gfx950).
//
// The quantizer is the per-token, per-128-element-group FP8 quantizer of
// the page "fp8_act_quant.rs" (module doc: one group of 128 K elements of
// one token at a time; `fp8_quant_grid`: tokens on grid X, K groups on Y).
// The page gives the grouping and the grids, not the arithmetic; the
// arithmetic here is the plainest reading, the same rule as the weight
// blocks' scales: per (token, group) s = amax / 448 in FP32 (448 is the
// largest E4M3 value), code = E4M3 round-to-nearest-even of x / s in FP32,
// saturated to +-448; an all-zero group gets s = 0 and zero codes.
//
//   * One thread owns 8 consecutive elements (one 16-byte load of BF16);
//     16 threads own a group and reduce its amax with lane shuffles; a
//     256-thread workgroup covers 16 groups of one row.
//   * The FP32 -> E4M3 conversion is the hardware's (v_cvt_pk_fp8_f32,
//     OCP E4M3FN, round to nearest even); inputs are clamped to +-448
//     first, so it never sees an out-of-range value.
//
// The W8A8 GEMM is the W8A16 operation with A given as FP8 codes and one
// FP32 scale per (row, 128-wide K step):
//     C[i, j] = bf16( sum_b Sa[i, b] * Sw[j / 128, b] *
//                      sum_t Qa[i, 128b + t] * W[j, 128b + t] )
// It follows the stream kernel's organisation (a workgroup owns NBW 16-column
// and MB 16-row blocks of C over all of K, its waves take interleaved K
// steps, the partial tiles are added in wave order) with two changes: A is
// staged exactly like the weight (16 rows x 128 bytes per block and step,
// same swizzle), and one v_mfma 16x16x128 FP8 x FP8 instruction covers a
// whole K step, so there is no dequantization at all.  The step's partial
// is folded with the product of the two scales: acc = fma(sa * sw, p, acc).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

using namespace dev;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr uint32_t kBlk = 2048;   // LDS bytes of one 16-row FP8 block per K step

// ---------------------------------------------------------------- quantizer

__global__ __launch_bounds__(256) void w8a16_act_quant_kernel(QuantArgs q)
{
    const uint32_t row = blockIdx.x;
    const uint32_t groups = q.k / 128u;
    const uint32_t g = blockIdx.y * 16u + (threadIdx.x >> 4);
    const uint32_t sub = threadIdx.x & 15u;
    if (g >= groups)
        return;   // whole 16-lane groups leave together
    const uint16_t *src = reinterpret_cast<const uint16_t *>(q.a) + (size_t)row * q.a_stride +
                          g * 128u + sub * 8u;
    const u32x4_t raw = *reinterpret_cast<const u32x4_t *>(src);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float s = __fdiv_rn(amax, 448.0f);
    u32x2_t codes = {0u, 0u};
    if (s != 0.f) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            y[i] = fminf(fmaxf(__fdiv_rn(x[i], s), -448.0f), 448.0f);
        int lo = 0, hi = 0;
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], lo, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], hi, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
        codes.x = (uint32_t)lo;
        codes.y = (uint32_t)hi;
    }
    *reinterpret_cast<u32x2_t *>(q.q + (size_t)row * q.q_stride + g * 128u + sub * 8u) = codes;
    if (sub == 0)
        q.scales[(size_t)row * groups + g] = s;
}

// ---------------------------------------------------------------- W8A8 GEMM

// NTW: load the weight with the non-temporal hint (one row tile: each
// weight byte is read once).  Measured on MI355X, us per call, hint vs
// plain loads: 16 x 12288 x 5120 13.0-13.3 vs 14.4-14.7, but 8 x 4096 x
// 4096 (16 MiB) 5.57-5.59 vs 5.43-5.49, so only weights above 16 MiB take it.
template <int MB, int NBW, int WAVES, bool NTW>
__device__ __forceinline__ void w8a8_tile(const GemmArgs &g, const float *a_scales)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int DEPTH = 2;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tile = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t m_tile = tile % g.m_tiles;
    const uint32_t n_tile = tile / g.m_tiles;
    const uint32_t n0 = n_tile * (NBW * 16);
    const uint32_t m0 = m_tile * (MB * 16);
    const uint32_t ksteps = g.k / 128u;
    // This wave's K steps: wave, wave + WAVES, ... (nw of them), walked from
    // a per-tile rotation so that neighbouring tiles read different K.
    const uint32_t nw = wave < ksteps ? (ksteps - wave + WAVES - 1) / WAVES : 0u;
    const uint32_t rot = (tile * kRotStride) % ksteps;
    auto phys = [&](uint32_t i) {
        uint32_t x = i + rot;
        return x >= ksteps ? x - ksteps : x;
    };

    uint8_t *wl = lds + wave * ((NBW + MB) * kBlk);
    uint8_t *al = wl + NBW * kBlk;
    const uint32_t rr = lane & 15u, gq = lane >> 4;

    // Coalesced loads: weight / A row 8h + lane/8 of each 16-row block,
    // 16-byte chunk lane%8, stored swizzled; read back in MFMA layout (row
    // rr, chunks 2gq and 2gq + 1: lane group gq takes K bytes 32gq..32gq+31
    // of the step from both operands).  Rows past n or m read the last
    // valid row; their outputs are never stored.
    const uint8_t *wsrc[NBW][2];
    const uint8_t *asrc[MB][2];
    uint32_t dst[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t r = 8u * h + (lane >> 3);
        dst[h] = r * 128u + (((lane & 7u) ^ wswz(r)) * 16u);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            wsrc[j][h] = g.w + (size_t)min(n0 + 16u * j + r, g.n - 1u) * g.k + (lane & 7u) * 16u;
#pragma unroll
        for (int b = 0; b < MB; ++b)
            asrc[b][h] = g.a + (size_t)min(m0 + 16u * b + r, g.m - 1u) * g.a_stride +
                         (lane & 7u) * 16u;
    }
    const uint32_t rd0 = rr * 128u + (((2u * gq) ^ wswz(rr)) * 16u);
    const uint32_t rd1 = rr * 128u + (((2u * gq + 1u) ^ wswz(rr)) * 16u);
    const float *srow[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
        srow[j] = g.scale + (size_t)(min(n0 + 16u * j, g.n - 1u) / 128u) * ksteps;
    // The A scale of this lane's output row in each 16-row block.
    const float *arow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        arow[b] = a_scales + (size_t)min(m0 + 16u * b + rr, g.m - 1u) * ksteps;

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wr[DEPTH][NBW][2];
    u32x4_t ar[DEPTH][MB][2];
    float sw[DEPTH][NBW];
    float sa[DEPTH][MB];
    auto issue = [&](int d, uint32_t t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                wr[d][j][h] = NTW ? __builtin_nontemporal_load(
                                        reinterpret_cast<const u32x4_t *>(wsrc[j][h] + t * 128u))
                                  : *reinterpret_cast<const u32x4_t *>(wsrc[j][h] + t * 128u);
#pragma unroll
            for (int b = 0; b < MB; ++b)
                ar[d][b][h] = *reinterpret_cast<const u32x4_t *>(asrc[b][h] + t * 128u);
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            sw[d][j] = srow[j][t];
#pragma unroll
        for (int b = 0; b < MB; ++b)
            sa[d][b] = arow[b][t];
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if ((uint32_t)d < nw)
            issue(d, phys(wave + WAVES * d));

    for (uint32_t base = 0; base < nw; base += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint32_t i = base + d;
            if (i >= nw)
                break;
            float cw[NBW], ca[MB];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < NBW; ++j)
                    *reinterpret_cast<u32x4_t *>(wl + j * kBlk + dst[h]) = wr[d][j][h];
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    *reinterpret_cast<u32x4_t *>(al + b * kBlk + dst[h]) = ar[d][b][h];
            }
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                cw[j] = sw[d][j];
#pragma unroll
            for (int b = 0; b < MB; ++b)
                ca[b] = sa[d][b];
            if (i + DEPTH < nw)
                issue(d, phys(wave + WAVES * (i + DEPTH)));
            // The wave's own LDS area: its writes above are visible to its
            // own reads below (LDS operations of a wave complete in order).
            i32x8_t aop[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const u32x4_t x0 = *reinterpret_cast<const u32x4_t *>(al + b * kBlk + rd0);
                const u32x4_t x1 = *reinterpret_cast<const u32x4_t *>(al + b * kBlk + rd1);
                aop[b] = i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                 (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            }
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const u32x4_t x0 = *reinterpret_cast<const u32x4_t *>(wl + j * kBlk + rd0);
                const u32x4_t x1 = *reinterpret_cast<const u32x4_t *>(wl + j * kBlk + rd1);
                const i32x8_t wop = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    // formats 0/0: both operands E4M3; block scales 2^0
                    const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wop, aop[b], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                    const float s = ca[b] * cw[j];
                    acc[j][b].x = __builtin_fmaf(s, p.x, acc[j][b].x);
                    acc[j][b].y = __builtin_fmaf(s, p.y, acc[j][b].y);
                    acc[j][b].z = __builtin_fmaf(s, p.z, acc[j][b].z);
                    acc[j][b].w = __builtin_fmaf(s, p.w, acc[j][b].w);
                }
            }
        }
    }

    // ---- add the waves' partial tiles in wave order ----------------------
    constexpr int P = NBW * MB;
    __syncthreads();
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            red[(wave * P + j * MB + b) * 64 + lane] = acc[j][b];
    __syncthreads();
    if constexpr (P < WAVES) {
        // Fewer output tiles than waves: every thread adds one output's
        // partials, in wave order.
        constexpr uint32_t F = P * 256u;
        const float *redf = reinterpret_cast<const float *>(lds);
        for (uint32_t f = threadIdx.x; f < F; f += WAVES * 64u) {
            float v[WAVES];
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                v[w] = redf[w * F + f];
            float sum = v[0];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                sum += v[w];
            const uint32_t pi = f / 256u, ln = (f % 256u) / 4u;
            const uint32_t j = pi / MB, b = pi % MB;
            const uint32_t row = m0 + 16u * b + (ln & 15u);
            const uint32_t col = n0 + 16u * j + 4u * (ln >> 4) + f % 4u;
            if (row < g.m && col < g.n)
                reinterpret_cast<uint16_t *>(g.c)[(size_t)row * g.c_stride + col] =
                    (uint16_t)f32_to_bf16_bits(sum);
        }
    } else {
        for (uint32_t pi = wave; pi < (uint32_t)P; pi += WAVES) {
            f32x4_t s = red[pi * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                s += red[(w * P + pi) * 64 + lane];
            const uint32_t j = pi / MB, b = pi % MB;
            store_c4(g, s, m0 + 16u * b + rr, n0 + 16u * j + 4u * gq);
        }
    }
}

// One instance per weight load form (chosen on the host), so the
// plain-load instance is not burdened by the hinted form's code.
template <int MB, int NBW, int WAVES, bool NTW>
__global__ __launch_bounds__(WAVES * 64) void w8a16_w8a8_kernel(GemmArgs g, const float *a_scales)
{
    w8a8_tile<MB, NBW, WAVES, NTW>(g, a_scales);
}

template <int MB, int NBW, bool NTW>
hipError_t launch_w8a8_mnt(const GemmArgs &g, const float *a_scales, const w8a16_plan_t &p,
                           hipStream_t stream)
{
    void (*kern)(GemmArgs, const float *);
    switch (p.waves) {
    case 4: kern = w8a16_w8a8_kernel<MB, NBW, 4, NTW>; break;
    case 8: kern = w8a16_w8a8_kernel<MB, NBW, 8, NTW>; break;
    case 16:
        // 16 waves fit the register budget (128 VGPRs) only with at most
        // two blocks per workgroup; the planner never asks for more.
        if constexpr (MB * NBW <= 2)
            kern = w8a16_w8a8_kernel<MB, NBW, 16, NTW>;
        else
            return hipErrorInvalidValue;
        break;
    default: return hipErrorInvalidValue;
    }
    // one flag set per (MB, NBW, NTW) instantiation, covering its three wave counts
    static std::atomic<uint64_t> lds_set[3];
    const int wi = p.waves == 4 ? 0 : (p.waves == 8 ? 1 : 2);
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), p.lds_bytes, kMaxLdsBytes,
                             lds_set[wi]);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g, a_scales);
    return hipGetLastError();
}

template <int MB, int NBW>
hipError_t launch_w8a8_mn(const GemmArgs &g, const float *a_scales, const w8a16_plan_t &p,
                          hipStream_t stream)
{
    if (g.m_tiles == 1 && (uint64_t)g.n * g.k > (16ull << 20))
        return launch_w8a8_mnt<MB, NBW, true>(g, a_scales, p, stream);
    return launch_w8a8_mnt<MB, NBW, false>(g, a_scales, p, stream);
}

}  // namespace

hipError_t launch_act_quant(const QuantArgs &q, hipStream_t stream)
{
    const uint32_t groups = q.k / 128u;
    hipLaunchKernelGGL(w8a16_act_quant_kernel, dim3(q.m, (groups + 15u) / 16u), dim3(256), 0,
                       stream, q);
    return hipGetLastError();
}

hipError_t launch_w8a8(const GemmArgs &g, const float *a_scales, const w8a16_plan_t &p,
                       hipStream_t stream)
{
    switch (p.m_blocks * 100 + p.n_blocks) {
    case 101: return launch_w8a8_mn<1, 1>(g, a_scales, p, stream);
    case 102: return launch_w8a8_mn<1, 2>(g, a_scales, p, stream);
    case 103: return launch_w8a8_mn<1, 3>(g, a_scales, p, stream);
    case 104: return launch_w8a8_mn<1, 4>(g, a_scales, p, stream);
    case 201: return launch_w8a8_mn<2, 1>(g, a_scales, p, stream);
    case 202: return launch_w8a8_mn<2, 2>(g, a_scales, p, stream);
    case 204: return launch_w8a8_mn<2, 4>(g, a_scales, p, stream);
    case 401: return launch_w8a8_mn<4, 1>(g, a_scales, p, stream);
    case 402: return launch_w8a8_mn<4, 2>(g, a_scales, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w8a16
