// Wide-tile W8A16 GEMM kernel for 65..128-row (and taller) GEMMs over large
// weights (gfx950).
//
// Same operation as the other kernels (page "w8a16_gemm_pipelined_m32.rs":
// operand layouts in the doc comment of `w8a16_gemm_pipelined_m32_strided`,
// one FP32 scale per 128x128 weight block folded once per 128-wide K step,
// `W8A16_M32_K_BLOCK`; the 128-row tile that shares the dequantized weight
// across all its rows is the page's large-row path,
// `w8a16_gemm_pipelined_by_m`).
//
// What bounds the 64 x 128 tile kernel at 128 rows is the bytes each CU pulls
// through its L1 (A rows and weight rows of its tile, per K) and the LDS
// bytes its waves read per MFMA.  This kernel takes both down:
//
//   * A workgroup owns a 128 x 256 tile of C (all of a 128-row M, so every
//     weight byte crosses HBM once) over a range of 128-wide K steps; K is
//     split so the tiles fill the CUs.  Per K column a CU requests 2 * 128
//     bytes of A and 256 of weight: half of what two 64 x 128 tiles need.
//   * 4 waves, one per SIMD, each owning a 64-row x 128-column quarter as
//     2 x 4 blocks of v_mfma_f32_32x32x16_bf16: per 16 K a wave reads 64
//     rows of A (BF16) and 128 of weight (FP8) from LDS for 8 MFMAs, 256
//     LDS bytes per 16K flops instead of 512 for 32 x 64 quarters.
//   * The FP8 weight goes straight from global memory into LDS with
//     global_load_lds_dwordx4, a ring of 3 K steps (two ahead: it comes from
//     HBM); A in a ring of 3 half steps (64 K each; it comes from L2).  Each
//     lane picks the 16 bytes it moves so that the LDS image is XOR-swizzled
//     in 128-byte rows while 8 lanes still read one whole 128-byte line.
//     Waves 0 and 1 issue the weight ring, waves 2 and 3 the A ring and the
//     scale rows, so each wave's vmcnt waits cover only its own ring.
//   * Inside a K step the MFMA's K index is a free relabelling of the
//     physical k: for half h, lane group g (= lane / 32) and 16-K slice s,
//     the lanes take physical k 64h + 32g + 8s .. +7 of the step from both
//     operands, so a lane reads 32 contiguous weight bytes and 64
//     contiguous A bytes per half.
//   * The weight is dequantized after the LDS read, exactly, with
//     v_cvt_scalef32_pk_bf16_fp8 at scale 1.0.
//   * Each step's 16 MFMA partials per block start at zero and are folded
//     into the FP32 accumulator with the step's block scale:
//     acc = fma(s, partial, acc).  A wave's 128 columns are one 128-row
//     scale block, so the scale is one value per step.
//   * With a K split each workgroup stores its FP32 tile and the split
//     reduction kernel adds the splits in split order.
//   * Rows past m and columns past n are read from clamped, valid
//     addresses and never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

using namespace dev;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr uint32_t kMT = 128;                 // C rows per tile
constexpr uint32_t kNT = 256;                 // C columns per tile
constexpr int kWST = 3;                       // weight ring: 128-wide K steps
constexpr int kAST = 3;                       // A ring: 64-wide K halves
constexpr uint32_t kWStep = kNT * 128;        // one K step of weight: 32 KiB
constexpr uint32_t kAHalf = kMT * 128;        // one K half of A: 16 KiB
constexpr int kWLoads = kWStep / 1024 / 2;    // 1 KiB DMA loads per weight wave per step
constexpr int kALoads = kAHalf / 1024 / 2;    // per A wave per half

static_assert(wide_lds_bytes() == kWST * kWStep + kAST * kAHalf + 2 * 256,
              "LDS layout of the wide kernel");

// One K step of the weight into an LDS buffer: this wave's kWLoads of the
// step's 32 loads (8 rows of 128 bytes each).  Lane i of load u writes slot
// i % 8 of row 8u + i / 8, so it reads the chunk that slot holds.
template <int AUX>
__device__ __forceinline__ void issue_w(uint8_t *dst, uint32_t t, const GemmArgs &g, uint32_t n0,
                                        uint32_t grp, uint32_t lane)
{
#pragma unroll
    for (int j = 0; j < kWLoads; ++j) {
        const uint32_t u = grp * kWLoads + j;
        const uint32_t r = 8u * u + (lane >> 3);
        const uint32_t c = (lane & 7u) ^ wswz(r & 15u);
        const uint32_t row = min(n0 + r, g.n - 1u);
        __builtin_amdgcn_global_load_lds(g.w + (size_t)row * g.k + t * 128u + c * 16u,
                                         (lds_void_t *)(dst + u * 1024u), 16, 0, AUX);
    }
}

// One K half (64 K = 128 bytes of each A row) of A into an LDS buffer.
__device__ __forceinline__ void issue_a(uint8_t *dst, uint32_t hs, uint32_t s0,
                                        const GemmArgs &g, uint32_t m0, uint32_t grp,
                                        uint32_t lane)
{
    const uint32_t byte0 = (s0 + hs / 2u) * 256u + (hs & 1u) * 128u;
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
        const uint32_t u = grp * kALoads + j;
        const uint32_t r = 8u * u + (lane >> 3);
        const uint32_t c = (lane & 7u) ^ wswz(r & 15u);
        const uint32_t row = min(m0 + r, g.m - 1u);
        __builtin_amdgcn_global_load_lds(g.a + (size_t)row * g.a_stride * 2u + byte0 + c * 16u,
                                         (lds_void_t *)(dst + u * 1024u), 16, 0, 0);
    }
}

// s_waitcnt vmcnt(PER * ahead) for a wave-uniform ahead in 0..MAXA.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_ahead(uint32_t ahead)
{
    if constexpr (MAXA <= 0) {
        wait_vm<0>();
    } else {
        if (ahead >= (uint32_t)MAXA)
            wait_vm<PER * MAXA>();
        else
            wait_ahead<PER, MAXA - 1>(ahead);
    }
}

// 8 FP8 bytes (two dwords) -> one 32x32x16 operand of 8 BF16.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t x, uint32_t y)
{
    u32x4_t v;
    v.x = bf16_pair_from_fp8<false>(x);
    v.y = bf16_pair_from_fp8<true>(x);
    v.z = bf16_pair_from_fp8<false>(y);
    v.w = bf16_pair_from_fp8<true>(y);
    return __builtin_bit_cast(bf16x8_t, v);
}

// NTW: the weight's DMA carries the non-temporal hint (one row tile reads
// each weight byte once; the host picks the instance).
template <bool NTW>
__global__ __launch_bounds__(256) void w8a16_wide_kernel(GemmArgs g)
{
    constexpr int WAUX = NTW ? kNonTemporal : 0;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *const wbuf = lds;
    uint8_t *const abuf = lds + kWST * kWStep;
    float *const scl = reinterpret_cast<float *>(abuf + kAST * kAHalf);   // [2][64]

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave & 1u, wn = wave >> 1;
    const bool wrole = wave < 2u;             // weight ring, else A ring
    const uint32_t grp = wave & 1u;           // half of its ring's loads
    const uint32_t lid = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t split = lid % g.splits;
    const uint32_t tile = lid / g.splits;
    const uint32_t m0 = (tile % g.m_tiles) * kMT;
    const uint32_t n0 = (tile / g.m_tiles) * kNT;
    const uint32_t ksteps = g.k / 128u;
    const uint32_t s0 = split * g.steps_per_split;
    const uint32_t s1 = min(ksteps, s0 + g.steps_per_split);
    const uint32_t nsteps = s1 - s0;          // >= 1 (the planner's splits are not empty)
    const uint32_t nhalves = 2u * nsteps;

    // ---- prologue: two weight steps, the scale rows and two A halves -----
    if (wrole) {
#pragma unroll
        for (int st = 0; st < kWST - 1; ++st)
            if ((uint32_t)st < nsteps)
                issue_w<WAUX>(wbuf + st * kWStep, s0 + st, g, n0, grp, lane);
    } else {
        if (grp == 0u) {
            // scale rows of the tile's two 128-column blocks for this split's
            // steps (at most 64, which the planner guarantees), lane l taking
            // step s0 + l; the first A wait covers them
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t nb = min(n0 + 128u * b, g.n - 1u) / 128u;
                __builtin_amdgcn_global_load_lds(
                    g.scale + (size_t)nb * ksteps + min(s0 + lane, s1 - 1u),
                    (lds_void_t *)(scl + 64 * b), 4, 0, 0);
            }
        }
#pragma unroll
        for (int hs = 0; hs < kAST - 1; ++hs)
            if ((uint32_t)hs < nhalves)
                issue_a(abuf + hs * kAHalf, hs, s0, g, m0, grp, lane);
    }

    // ---- per-lane LDS read offsets ------------------------------------------
    const uint32_t rr = lane & 31u, gq = lane >> 5;
    // A: row 64wm + 32bm + rr of a half buffer, chunk 4gq + s (slice s)
    uint32_t aoff[2][4];
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t r = 64u * wm + 32u * bm + rr;
            aoff[bm][s] = r * 128u + (((4u * gq + s) ^ wswz(r & 15u)) * 16u);
        }
    // weight: row 128wn + 32bn + rr of a step buffer, chunks 4h + 2gq + {0, 1}
    uint32_t woff[4][2][2];
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t r = 128u * wn + 32u * bn + rr;
                woff[bn][h][e] = r * 128u + (((4u * h + 2u * gq + e) ^ wswz(r & 15u)) * 16u);
            }

    f32x16_t acc[4][2];
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
            acc[bn][bm] = f32x16_t{};
    f32x16_t p[4][2];

    for (uint32_t idx = 0; idx < nsteps; ++idx) {
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t hs = 2u * idx + h;
            // Each issuing wave waits until only the loads it issued after
            // this step (weight) or half (A) are outstanding.
            if (wrole) {
                if (h == 0u)
                    wait_ahead<kWLoads, kWST - 2>(min((uint32_t)(kWST - 2), nsteps - 1u - idx));
            } else {
                wait_ahead<kALoads, kAST - 2>(min((uint32_t)(kAST - 2), nhalves - 1u - hs));
            }
            barrier_lds();
            // Every wave is past the previous half: refill the buffers it used.
            if (wrole) {
                if (h == 0u && idx + kWST - 1u < nsteps)
                    issue_w<WAUX>(wbuf + ((idx + kWST - 1u) % kWST) * kWStep,
                                  s0 + idx + kWST - 1u, g, n0, grp, lane);
            } else {
                if (hs + kAST - 1u < nhalves)
                    issue_a(abuf + ((hs + kAST - 1u) % kAST) * kAHalf, hs + kAST - 1u, s0, g,
                            m0, grp, lane);
            }

            const uint8_t *sa = abuf + (hs % kAST) * kAHalf;
            const uint8_t *sw = wbuf + (idx % kWST) * kWStep;
            u32x4_t wraw[4][2];
#pragma unroll
            for (int bn = 0; bn < 4; ++bn)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    wraw[bn][e] = *reinterpret_cast<const u32x4_t *>(sw + woff[bn][h][e]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8_t af[2];
#pragma unroll
                for (int bm = 0; bm < 2; ++bm)
                    af[bm] = *reinterpret_cast<const bf16x8_t *>(sa + aoff[bm][s]);
#pragma unroll
                for (int bn = 0; bn < 4; ++bn) {
                    const u32x4_t c = wraw[bn][s >> 1];
                    const bf16x8_t wb = (s & 1) ? dequant8(c.z, c.w) : dequant8(c.x, c.y);
#pragma unroll
                    for (int bm = 0; bm < 2; ++bm)
                        p[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            wb, af[bm], (h == 0u && s == 0) ? f32x16_t{} : p[bn][bm], 0, 0, 0);
                }
            }
        }
        const float sc = scl[64u * wn + idx];
#pragma unroll
        for (int bn = 0; bn < 4; ++bn)
#pragma unroll
            for (int bm = 0; bm < 2; ++bm)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[bn][bm][v] = __builtin_fmaf(sc, p[bn][bm][v], acc[bn][bm][v]);
    }

    // ---- epilogue: lane holds C[row][col..col+3] for each (bn, bm, q) -------
    // (32x32 MFMA result: register 4q + i of lane l is D[8q + 4(l/32) + i][l % 32],
    // with D's rows the weight rows, i.e. C columns.)
    const uint32_t row0 = m0 + 64u * wm + rr;
    const uint32_t col0 = n0 + 128u * wn + 4u * gq;
    if (g.splits == 1) {
#pragma unroll
        for (int bn = 0; bn < 4; ++bn)
#pragma unroll
            for (int bm = 0; bm < 2; ++bm)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16_t &a = acc[bn][bm];
                    store_c4(g, f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]},
                             row0 + 32u * bm, col0 + 32u * bn + 8u * q);
                }
        return;
    }
    // Workspace [splits][m_tiles * 128][n_tiles * 256] FP32, whole tiles.
    const size_t ws_cols = (size_t)g.n_tiles * kNT;
    float *wsp = g.ws + ((size_t)split * g.m_tiles * kMT) * ws_cols;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
        for (int bm = 0; bm < 2; ++bm)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x16_t &a = acc[bn][bm];
                *reinterpret_cast<f32x4_t *>(wsp + (size_t)(row0 + 32u * bm) * ws_cols + col0 +
                                             32u * bn + 8u * q) =
                    f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
            }
}

template <bool NTW>
hipError_t launch_wide_t(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    auto kern = w8a16_wide_kernel<NTW>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), p.lds_bytes, kMaxLdsBytes,
                             lds_set);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g);
    e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1)
        return e;
    return launch_split_reduce(g, p.n_tiles * kNT, p.m_tiles * kMT, stream);
}

}  // namespace

hipError_t launch_wide(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if (p.m_blocks != kMT / 16 || p.n_blocks != kNT / 16 || p.block != 256)
        return hipErrorInvalidValue;
    if (g.m_tiles == 1)
        return launch_wide_t<true>(g, p, stream);
    return launch_wide_t<false>(g, p, stream);
}

}  // namespace w8a16
