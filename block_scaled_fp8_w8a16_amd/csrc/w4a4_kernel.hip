// W4A4 MX projection GEMV kernels (gfx950).
//
// The m-row projection planned on the page "w4a4_proj/mx_plan.rs" (m up to
// 64; weight rows in 16-row tiles; the activation-reuse twins feed one
// activation fragment to several weight tiles; the persistent entry stages
// the activations once per workgroup and pulls 16-row tiles from a counter),
// with both operands in the OCP MXFP4 format: FP4 E2M1 elements, two per
// byte with the even element in the low nibble, one E8M0 scale per 32
// consecutive K elements of a row.
//
//   C[i][j] = bf16( sum_b 2^(ea[i][b] - 127) * 2^(ew[j][b] - 127) * sum_t a[i][32b+t] * w[j][32b+t] )
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes FP4 operands and one
// E8M0 scale per 32 K elements of each row and column, so a 128-wide K step
// of a 16 x 16 output block is one instruction with the block scales applied
// in hardware and FP32 accumulation; there is no dequantization and no scale
// fold.
//
//   * MFMA operand layout: lane l holds row l % 16 of a 16-row block and the
//     32 K elements 32 (l / 16) .. +31 of the step (16 bytes), which is one
//     MX block, so its scale byte is that lane's own.  A direct load in this
//     layout reads 16 rows x 64 contiguous bytes per instruction, the whole
//     step of each row, so the weight goes straight to registers (no LDS).
//   * Tiled kernel: a workgroup owns NBW 16-column blocks of C and MB 16-row
//     blocks over all of K; its waves take interleaved K steps, DEPTH steps
//     of loads in flight each; every A fragment feeds the NBW weight blocks
//     from registers.  The waves' partial tiles are added in LDS in wave
//     order, then stored as BF16.
//   * Persistent kernel (9..32 rows over a wide weight): one workgroup per
//     CU stages all of A and its scales in LDS once; each wave pulls 16-row
//     weight tiles from a counter and walks all of K for its tile alone, so
//     A is read from HBM/L2 once per CU instead of once per tile.  Every
//     wave stops at the first ticket past the last tile; the last workgroup
//     to finish puts the counters back to zero for the next call.
//   * Rows past m and columns past n read clamped, valid addresses and are
//     never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

using namespace dev;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Format operands of the scaled MFMA: 4 = FP4 E2M1 for both sources.
constexpr int kFmtFp4 = 4;

__device__ __forceinline__ i32x8_t fp4_operand(u32x4_t v)
{
    return i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// One 16x16 block's K step: acc += (W rows scaled) x (A rows scaled)^T.
__device__ __forceinline__ f32x4_t mx_step(u32x4_t w, uint32_t ws, u32x4_t a, uint32_t as,
                                           f32x4_t acc)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        fp4_operand(w), fp4_operand(a), acc, kFmtFp4, kFmtFp4, 0, (int)ws, 0, (int)as);
}

// Add the WAVES partial tiles of the workgroup in wave order and store C.
// red: LDS of WAVES * P * 1 KiB.
template <int MB, int NBW, int WAVES>
__device__ __forceinline__ void reduce_store(const MxArgs &g, f32x4_t (&acc)[NBW][MB],
                                             uint32_t m0, uint32_t n0, uint32_t wave,
                                             uint32_t lane)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int P = NBW * MB;
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            red[(wave * P + j * MB + b) * 64 + lane] = acc[j][b];
    __syncthreads();
    // every thread adds one output's partials, in wave order
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
        // float f is component f % 4 of lane (f % 256) / 4 of pair f / 256
        const uint32_t pi = f / 256u, ln = (f % 256u) / 4u;
        const uint32_t j = pi / MB, b = pi % MB;
        const uint32_t row = m0 + 16u * b + (ln & 15u);
        const uint32_t col = n0 + 16u * j + 4u * (ln >> 4) + f % 4u;
        if (row < g.m && col < g.n)
            reinterpret_cast<uint16_t *>(g.c)[(size_t)row * g.c_stride + col] =
                (uint16_t)f32_to_bf16_bits(sum);
    }
}

template <int MB, int NBW, int WAVES, int DEPTH, bool NTW>
__global__ __launch_bounds__(WAVES * 64) void w8a16_w4a4_kernel(MxArgs g)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tile = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t m0 = (tile % g.m_tiles) * (MB * 16);
    const uint32_t n0 = (tile / g.m_tiles) * (NBW * 16);
    const uint32_t ksteps = g.k / 128u;
    const uint32_t kb = g.k / 32u;                     // scale bytes per row
    const uint32_t rr = lane & 15u, gq = lane >> 4;
    // this wave's K steps: wave, wave + WAVES, ... (nw of them), walked from
    // a per-tile rotation so that neighbouring tiles read different K
    const uint32_t nw = wave < ksteps ? (ksteps - wave + WAVES - 1) / WAVES : 0u;
    const uint32_t rot = (tile * kRotStride) % ksteps;
    auto phys = [&](uint32_t i) {
        uint32_t x = wave + WAVES * i + rot;
        return x >= ksteps ? x - ksteps : x;
    };

    // per-lane operand addresses: row rr of each 16-row block, byte 16 gq of
    // the step's 64 bytes; the scale byte of that row and 32-element block
    const uint8_t *wsrc[NBW], *wsc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const uint32_t row = min(n0 + 16u * j + rr, g.n - 1u);
        wsrc[j] = g.w + (size_t)row * (g.k / 2u) + 16u * gq;
        wsc[j] = g.w_scale + (size_t)row * kb + gq;
    }
    const uint8_t *asrc[MB], *asc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const uint32_t row = min(m0 + 16u * b + rr, g.m - 1u);
        asrc[b] = g.a + (size_t)row * g.a_stride + 16u * gq;
        asc[b] = g.a_scale + (size_t)row * kb + gq;
    }

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wr[DEPTH][NBW], ar[DEPTH][MB];
    uint32_t wsr[DEPTH][NBW], asr[DEPTH][MB];
    auto issue = [&](int d, uint32_t t) {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const u32x4_t *p = reinterpret_cast<const u32x4_t *>(wsrc[j] + t * 64u);
            wr[d][j] = NTW ? __builtin_nontemporal_load(p) : *p;
            wsr[d][j] = wsc[j][t * 4u];
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            ar[d][b] = *reinterpret_cast<const u32x4_t *>(asrc[b] + t * 64u);
            asr[d][b] = asc[b][t * 4u];
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if ((uint32_t)d < nw)
            issue(d, phys(d));
    for (uint32_t base = 0; base < nw; base += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint32_t i = base + d;
            if (i >= nw)
                break;
            u32x4_t cw[NBW], ca[MB];
            uint32_t cws[NBW], cas[MB];
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                cw[j] = wr[d][j];
                cws[j] = wsr[d][j];
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                ca[b] = ar[d][b];
                cas[b] = asr[d][b];
            }
            if (i + DEPTH < nw)
                issue(d, phys(i + DEPTH));
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    acc[j][b] = mx_step(cw[j], cws[j], ca[b], cas[b], acc[j][b]);
        }
    }
    reduce_store<MB, NBW, WAVES>(g, acc, m0, n0, wave, lane);
}

// Persistent kernel: A (MB 16-row blocks, all of K) and its scales staged in
// LDS once; each wave pulls 16-row weight tiles from counters[0].
template <int MB, int WAVES, int DEPTH>
__global__ __launch_bounds__(WAVES * 64) void w8a16_w4a4_ps_kernel(MxArgs g)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ksteps = g.k / 128u;
    const uint32_t kb = g.k / 32u;
    const uint32_t pitch = g.k / 2u + 16u;            // LDS row pitch of A (bytes)
    uint8_t *alds = lds;                               // [MB * 16][pitch]
    uint8_t *slds = lds + MB * 16u * pitch;            // [MB * 16][kb]
    const uint32_t rr = lane & 15u, gq = lane >> 4;

    // stage A: 16-byte chunks of each of the MB * 16 rows (rows past m copy
    // the last valid row), then the scale bytes
    const uint32_t chunks = g.k / 32u;                 // 16-byte chunks per row
    for (uint32_t c = threadIdx.x; c < MB * 16u * chunks; c += WAVES * 64u) {
        const uint32_t r = c / chunks, q = c % chunks;
        const uint32_t row = min(r, g.m - 1u);
        *reinterpret_cast<u32x4_t *>(alds + r * pitch + q * 16u) =
            *reinterpret_cast<const u32x4_t *>(g.a + (size_t)row * g.a_stride + q * 16u);
    }
    for (uint32_t c = threadIdx.x; c < MB * 16u * kb; c += WAVES * 64u) {
        const uint32_t r = c / kb, q = c % kb;
        slds[c] = g.a_scale[(size_t)min(r, g.m - 1u) * kb + q];
    }
    __syncthreads();

    const uint32_t tiles = (g.n + 15u) / 16u;
    for (;;) {
        uint32_t t = 0;
        if (lane == 0)
            t = __hip_atomic_fetch_add(g.counters, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = __builtin_amdgcn_readfirstlane(t);
        if (t >= tiles)
            break;
        const uint32_t n0 = 16u * t;
        const uint32_t wrow = min(n0 + rr, g.n - 1u);
        const uint8_t *wsrc = g.w + (size_t)wrow * (g.k / 2u) + 16u * gq;
        const uint8_t *wsc = g.w_scale + (size_t)wrow * kb + gq;
        const uint32_t rot = (t * kRotStride) % ksteps;
        f32x4_t acc[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        u32x4_t wr[DEPTH];
        uint32_t wsr[DEPTH];
        auto phys = [&](uint32_t i) {
            uint32_t x = i + rot;
            return x >= ksteps ? x - ksteps : x;
        };
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if ((uint32_t)d < ksteps) {
                const uint32_t s = phys(d);
                wr[d] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(wsrc + s * 64u));
                wsr[d] = wsc[s * 4u];
            }
        for (uint32_t base = 0; base < ksteps; base += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const uint32_t i = base + d;
                if (i >= ksteps)
                    break;
                const uint32_t s = phys(i);
                const u32x4_t cw = wr[d];
                const uint32_t cws = wsr[d];
                if (i + DEPTH < ksteps) {
                    const uint32_t s2 = phys(i + DEPTH);
                    wr[d] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t *>(wsrc + s2 * 64u));
                    wsr[d] = wsc[s2 * 4u];
                }
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const uint32_t r = 16u * b + rr;
                    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(alds + r * pitch +
                                                                       s * 64u + 16u * gq);
                    const uint32_t as = slds[r * kb + s * 4u + gq];
                    acc[b] = mx_step(cw, cws, a, as, acc[b]);
                }
            }
        }
        // lane l holds C[row l % 16 of block b][n0 + 4 (l / 16) .. +3]
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const uint32_t row = 16u * b + rr;
            const uint32_t col = n0 + 4u * gq;
            if (row < g.m) {
                uint16_t *dst = reinterpret_cast<uint16_t *>(g.c) + (size_t)row * g.c_stride + col;
                const float v[4] = {acc[b].x, acc[b].y, acc[b].z, acc[b].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < g.n)
                        dst[e] = (uint16_t)f32_to_bf16_bits(v[e]);
            }
        }
    }
    // The last workgroup to finish puts both counters back to zero: by then
    // every wave has taken its final ticket.
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(g.counters + 1, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1u) {
            __hip_atomic_store(g.counters, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(g.counters + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <typename K>
hipError_t launch_mx(K kern, const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream,
                     std::atomic<uint64_t> &lds_set)
{
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), p.lds_bytes, kMaxLdsBytes,
                             lds_set);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g);
    return hipGetLastError();
}

template <int MB, int NBW, bool NTW>
hipError_t launch_w4a4_mnt(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    static std::atomic<uint64_t> lds_set[3];
    switch (p.waves) {
    case 4: return launch_mx(w8a16_w4a4_kernel<MB, NBW, 4, 2, NTW>, g, p, stream, lds_set[0]);
    case 8: return launch_mx(w8a16_w4a4_kernel<MB, NBW, 8, 2, NTW>, g, p, stream, lds_set[1]);
    case 16: return launch_mx(w8a16_w4a4_kernel<MB, NBW, 16, 2, NTW>, g, p, stream, lds_set[2]);
    default: return hipErrorInvalidValue;
    }
}

template <int MB, int NBW>
hipError_t launch_w4a4_mn(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if (g.m_tiles == 1)
        return launch_w4a4_mnt<MB, NBW, true>(g, p, stream);
    return launch_w4a4_mnt<MB, NBW, false>(g, p, stream);
}

template <int MB>
hipError_t launch_w4a4_ps_m(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    static std::atomic<uint64_t> lds_set[2];
    switch (p.waves) {
    case 8: return launch_mx(w8a16_w4a4_ps_kernel<MB, 8, 4>, g, p, stream, lds_set[0]);
    case 16: return launch_mx(w8a16_w4a4_ps_kernel<MB, 16, 4>, g, p, stream, lds_set[1]);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_w4a4(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if (p.kernel == W8A16_KERNEL_W4A4_PS) {
        switch (p.m_blocks) {
        case 1: return launch_w4a4_ps_m<1>(g, p, stream);
        case 2: return launch_w4a4_ps_m<2>(g, p, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.m_blocks * 100 + p.n_blocks) {
    case 101: return launch_w4a4_mn<1, 1>(g, p, stream);
    case 102: return launch_w4a4_mn<1, 2>(g, p, stream);
    case 104: return launch_w4a4_mn<1, 4>(g, p, stream);
    case 201: return launch_w4a4_mn<2, 1>(g, p, stream);
    case 202: return launch_w4a4_mn<2, 2>(g, p, stream);
    case 204: return launch_w4a4_mn<2, 4>(g, p, stream);
    case 401: return launch_w4a4_mn<4, 1>(g, p, stream);
    case 402: return launch_w4a4_mn<4, 2>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w8a16
