// Tiled W8A16 GEMM kernel for large m (gfx950), plus the fixed-order
// reduction of its K splits.  Included by tile_m64.hip and tile_m128.hip,
// which instantiate the 64-row and the 128-row variants in separate
// translation units (they build in parallel).
//
// Same operation as the stream kernel (page "w8a16_gemm_pipelined_m32.rs":
// operand layouts in the doc comment of `w8a16_gemm_pipelined_m32_strided`,
// one FP32 scale per 128x128 weight block folded once per 128-wide K step,
// `W8A16_M32_K_BLOCK`).  The page's large-row path is a 128-row tile that
// shares the dequantized weight across all its rows
// (`w8a16_gemm_pipelined_by_m`); this is that idea rebuilt for MI355X:
//
//   * A workgroup (4 waves, 2 x 2) owns an MT-row x NT-column tile of C
//     (MT, NT = 64 or 128) over a range of 128-wide K steps.  Each wave owns
//     MT/2 rows x NT/2 columns: MT/32 x NT/32 MFMA 16x16x32 tiles.
//   * Per K step the workgroup stages A (MT rows x 256 bytes of BF16) and
//     the weight (NT rows x 128 bytes of FP8) straight from global memory
//     into LDS with global_load_lds_dwordx4: the weight in a ring of WST
//     buffers (WST - 1 steps ahead, to cover HBM latency), A in a ring of
//     AST buffers (AST - 1 steps ahead; it comes from L2).
//     Each lane picks the 16 bytes it moves so that the LDS image comes out
//     XOR-swizzled in 128-byte rows (conflict-free MFMA operand reads) while
//     every 8 lanes still read one whole 128-byte line.  The compiler does not track
//     these DMA writes, so the kernel waits for them itself (s_waitcnt
//     vmcnt) and a workgroup barrier per step publishes them and retires
//     the buffers being refilled.
//   * vmcnt counts a wave's loads in issue order, so a wave that issued both
//     rings would, waiting for the near A step, also wait for every weight
//     step issued before it, and the weight ring would in effect be two
//     steps deep.  Loads are therefore split by wave: the even waves issue
//     the weight ring, the odd waves the A ring (and the scale row), and
//     each waits only for its own ring.
//   * The weight is dequantized after the LDS read (FP8 halves LDS traffic),
//     exactly, with v_cvt_scalef32_pk_bf16_fp8 at scale 1.0.
//   * Each step's MFMA partial starts at zero and is folded into the FP32
//     accumulator with the step's block scale: acc = fma(s, partial, acc).
//     An NT <= 128 tile aligned to NT never straddles two 128-row scale
//     blocks, so the scale is one scalar per step.
//   * Without a K split the workgroup stores BF16 C directly.  With splits,
//     it stores its FP32 tile to a workspace and a second kernel adds the
//     splits in split order: the kernel boundary publishes the partials,
//     where an in-kernel agent-scope release would cost an L2 writeback
//     per workgroup on this GPU.
//   * Rows past m and columns past n are read from clamped, valid addresses
//     and never stored.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

using namespace dev;


// DMA one K step of A, or of the weight, of this wave's share into an LDS
// buffer: loads u = 0..N-1 of the wave's group g, each one 1 KiB of LDS.
// __device__ functions rather than lambdas: a lambda in a kernel is also
// compiled for the host, where the DMA builtin does not exist.
// AUX: cache-policy operand (kNonTemporal for a weight read once).
template <int N, uint32_t STEP_BYTES, int AUX = 0>
__device__ __forceinline__ void issue_ring(uint8_t *dst, uint32_t grp, uint32_t t,
                                           const uint8_t *const *src)
{
#pragma unroll
    for (int u = 0; u < N; ++u)
        __builtin_amdgcn_global_load_lds(src[u] + t * STEP_BYTES,
                                         (lds_void_t *)(dst + (grp * N + u) * 1024u), 16, 0, AUX);
}

// Producer-wave forms: the whole ring's loads of one step, each address
// computed at issue (a producer has no math to overlap, and keeping 32
// pointers live would cost the compute waves registers).  Same LDS image as
// the shared forms: A load i fills plane i / (MT/8), rows 8(i % (MT/8))..+7; weight
// load i fills rows 8i..8i+7; lane s writes slot s % 8 of row s / 8.
template <int N, int MT>
__device__ __forceinline__ void issue_a_all(uint8_t *dst, uint32_t t, const GemmArgs &g,
                                            uint32_t m0, uint32_t lane)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t plane = (uint32_t)i / (MT / 8);
        const uint32_t r = 8u * ((uint32_t)i % (MT / 8)) + (lane >> 3);
        const uint32_t c = 8u * plane + ((lane & 7u) ^ wswz(r & 15u));
        const uint32_t row = min(m0 + r, g.m - 1u);
        __builtin_amdgcn_global_load_lds(g.a + (size_t)row * g.a_stride * 2u + c * 16u + t * 256u,
                                         (lds_void_t *)(dst + i * 1024u), 16, 0, 0);
    }
}

template <int N, int AUX>
__device__ __forceinline__ void issue_w_all(uint8_t *dst, uint32_t t, const GemmArgs &g,
                                            uint32_t n0, uint32_t lane)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t r = 8u * (uint32_t)i + (lane >> 3);
        const uint32_t c = (lane & 7u) ^ wswz(r & 15u);
        const uint32_t row = min(n0 + r, g.n - 1u);
        __builtin_amdgcn_global_load_lds(g.w + (size_t)row * g.k + c * 16u + t * 128u,
                                         (lds_void_t *)(dst + i * 1024u), 16, 0, AUX);
    }
}

// s_waitcnt vmcnt(PER * ahead) for a wave-uniform ahead in 0..MAXA.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_vm_ahead(uint32_t ahead)
{
    if constexpr (MAXA <= 0) {
        wait_vm<0>();
    } else {
        if (ahead >= (uint32_t)MAXA)
            wait_vm<PER * MAXA>();
        else
            wait_vm_ahead<PER, MAXA - 1>(ahead);
    }
}

// NTW: the weight's DMA carries the non-temporal hint (one row tile reads
// each weight byte once; the host picks the instance).
template <int MT, int NT, int WST, int AST, int KH, bool PROD, bool NTW>
__global__ __launch_bounds__(64 * (4 * KH + (PROD ? 2 : 0))) void w8a16_tile_kernel(GemmArgs g)
{
    constexpr int WAUX = NTW ? kNonTemporal : 0;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr uint32_t kABytes = MT * 256;   // one K step of A in LDS
    constexpr uint32_t kWBytes = NT * 128;
    constexpr int MBW = MT / 32;             // 16-row blocks per wave
    constexpr uint32_t CW = 4 * KH;          // compute waves
    // Loads per issuing wave per step: with PROD one producer wave issues a
    // whole ring, else the even compute waves share the weight ring and the
    // odd ones the A ring.
    constexpr int NA = kABytes / 1024 / (PROD ? 1 : 2 * KH);
    constexpr int NW = kWBytes / 1024 / (PROD ? 1 : 2 * KH);
    constexpr int QW = 4 / KH;               // MFMA k-quarters of a step per wave
    constexpr int HW = 2 / KH;               // 16-byte weight chunks per row per wave
    constexpr int NS = PROD ? 1 : (NA > NW ? NA : NW);
    // LDS: AST A buffers, WST weight buffers, the split's scale row.
    uint8_t *const abuf = lds;
    uint8_t *const wbuf = lds + AST * kABytes;
    float *const scl = reinterpret_cast<float *>(lds + AST * kABytes + WST * kWBytes);
    constexpr int NBW = NT / 32;             // 16-column blocks per wave
    static_assert(NW >= 1 && NBW >= 1 && AST >= 2 && WST >= 2, "tile too small");

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave & 1u, wn = (wave >> 1) & 1u;
    const uint32_t kh = (wave >> 2) & 1u;    // which k-quarters of each step (KH == 2)
    const bool computes = !PROD || wave < CW;
    const bool issues = !PROD || wave >= CW;
    const bool wrole = PROD ? wave == CW : (wave & 1u) == 0;   // weight ring, else A ring
    const uint32_t grp = PROD ? 0u : wave >> 1;                // share of its ring's loads
    const bool scale_wave = wave == (PROD ? CW + 1 : 1u);
    const uint32_t lid = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t split = lid % g.splits;
    const uint32_t tile = lid / g.splits;
    const uint32_t m_tile = tile % g.m_tiles;
    const uint32_t n_tile = tile / g.m_tiles;
    const uint32_t m0 = m_tile * MT;
    const uint32_t n0 = n_tile * NT;
    const uint32_t ksteps = g.k / 128u;
    const uint32_t s0 = split * g.steps_per_split;
    const uint32_t s1 = min(ksteps, s0 + g.steps_per_split);
    // All tiles of a split walk its K steps in the same order, so the tiles
    // sharing an L2 read each A step at about the same time and only the
    // first misses.  (Rotating the walk per tile, as the small-m kernels do
    // to spread weight reads over HBM channels, measured slower here: with
    // 512 KiB of weight streaming through each L2 per step, A steps read far
    // apart are evicted in between.)
    auto phys = [](uint32_t t) { return t; };

    // ---- DMA sources.  In LDS, A is two planes (K-step bytes 0..127 and
    // 128..255 of each row), each MT rows x 128 bytes; the weight is NT rows
    // x 128 bytes.  Within a 128-byte row r, slot p holds 16-byte chunk
    // p ^ wswz(r % 16): with rows 128 bytes apart this makes the MFMA operand
    // reads below (16 lanes = 16 consecutive rows, one chunk each) free of
    // LDS bank conflicts on gfx950, which 256-byte rows are not.  A DMA
    // instruction fills 1 KiB of LDS = 8 rows of one plane; lane s writes
    // slot s % 8 of row s / 8, so it reads the chunk that slot holds.
    const uint8_t *src[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        if (PROD || !issues) {
            src[u] = g.w;
        } else if (!wrole && u < NA) {
            const uint32_t i = grp * NA + u;          // plane i / (MT/8), rows 8(i % (MT/8))..+7
            const uint32_t plane = i / (MT / 8);
            const uint32_t r = 8u * (i % (MT / 8)) + (lane >> 3);
            const uint32_t c = 8u * plane + ((lane & 7u) ^ wswz(r & 15u));
            const uint32_t row = min(m0 + r, g.m - 1u);
            src[u] = g.a + (size_t)row * g.a_stride * 2u + c * 16u;
        } else if (wrole && u < NW) {
            const uint32_t i = grp * NW + u;          // rows 8i..8i+7
            const uint32_t r = 8u * i + (lane >> 3);
            const uint32_t c = (lane & 7u) ^ wswz(r & 15u);
            const uint32_t row = min(n0 + r, g.n - 1u);
            src[u] = g.w + (size_t)row * g.k + c * 16u;
        } else {
            src[u] = g.w;
        }
    }
    // ---- MFMA operand reads: row rr = lane % 16 of a 16-row block, lane
    // group gq = lane / 16 covers physical k 32gq..32gq+31 of the step (MFMA
    // q takes k 32gq+8q..+7 from both operands).
    const uint32_t rr = lane & 15u, gq = lane >> 4;
    // With KH == 2 the two groups of four waves take k-quarters 0-1 and 2-3
    // of every step over the same staged buffers, so each SIMD runs two
    // waves: one wave's LDS and barrier waits overlap the other's MFMAs.
    uint32_t aoff[MBW][QW];
#pragma unroll
    for (int b = 0; b < MBW; ++b)
#pragma unroll
        for (int qq = 0; qq < QW; ++qq) {
            const uint32_t q = kh * QW + qq;
            aoff[b][qq] = ((4u * gq + q) >> 3) * (MT * 128u) +
                          ((MT / 2) * wm + 16u * b + rr) * 128u +
                          ((((4u * gq + q) & 7u) ^ wswz(rr)) * 16u);
        }
    uint32_t woff[NBW][HW];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            const uint32_t h = kh * HW + hh;
            woff[j][hh] = ((NT / 2) * wn + 16u * j + rr) * 128u +
                          (((2u * gq + h) ^ wswz(rr)) * 16u);
        }
    f32x4_t acc[NBW][MBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MBW; ++b)
            acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Prologue.  Wave 1 first moves the scales of the tile's 128-row block
    // for this split's steps (at most 64, which the planner guarantees) into
    // LDS, lane l taking step s0 + l; its first wait covers them.
    if (!issues) {
    } else if (wrole) {
#pragma unroll
        for (int st = 0; st < WST - 1; ++st)
            if (s0 + st < s1) {
                if constexpr (PROD)
                    issue_w_all<NW, WAUX>(wbuf + st * kWBytes, phys(s0 + st), g, n0, lane);
                else
                    issue_ring<NW, 128u, WAUX>(wbuf + st * kWBytes, grp, phys(s0 + st), src);
            }
    } else {
        if (scale_wave && s0 < s1) {
            const float *srow = g.scale + (size_t)(min(n0, g.n - 1u) / 128u) * ksteps;
            __builtin_amdgcn_global_load_lds(srow + min(s0 + lane, s1 - 1u),
                                             (lds_void_t *)scl, 4, 0, 0);
        }
#pragma unroll
        for (int st = 0; st < AST - 1; ++st)
            if (s0 + st < s1) {
                if constexpr (PROD)
                    issue_a_all<NA, MT>(abuf + st * kABytes, phys(s0 + st), g, m0, lane);
                else
                    issue_ring<NA, 256u>(abuf + st * kABytes, grp, phys(s0 + st), src);
            }
    }

    for (uint32_t t = s0; t < s1; ++t) {
        const uint32_t idx = t - s0;
        // An issuing wave's ring holds min(RING - 2, s1 - 1 - t) steps issued
        // after step t; wait until only those are outstanding.
        if (issues) {
            if (wrole)
                wait_vm_ahead<NW, WST - 2>(min((uint32_t)(WST - 2), s1 - 1u - t));
            else
                wait_vm_ahead<NA, AST - 2>(min((uint32_t)(AST - 2), s1 - 1u - t));
        }
        barrier_lds();
        // Every wave is past step t - 1: refill the buffers it used.
        if (issues) {
            if (wrole) {
                if (t + WST - 1 < s1) {
                    uint8_t *dst = wbuf + ((idx + WST - 1) % WST) * kWBytes;
                    if constexpr (PROD)
                        issue_w_all<NW, WAUX>(dst, phys(t + WST - 1), g, n0, lane);
                    else
                        issue_ring<NW, 128u, WAUX>(dst, grp, phys(t + WST - 1), src);
                }
            } else {
                if (t + AST - 1 < s1) {
                    uint8_t *dst = abuf + ((idx + AST - 1) % AST) * kABytes;
                    if constexpr (PROD)
                        issue_a_all<NA, MT>(dst, phys(t + AST - 1), g, m0, lane);
                    else
                        issue_ring<NA, 256u>(dst, grp, phys(t + AST - 1), src);
                }
            }
        }
        if (!computes)
            continue;

        const uint8_t *sa = abuf + (idx % AST) * kABytes;
        const uint8_t *sw = wbuf + (idx % WST) * kWBytes;
        const float s = scl[phys(t) - s0];
        u32x4_t wraw[NBW][HW];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int hh = 0; hh < HW; ++hh)
                wraw[j][hh] = *reinterpret_cast<const u32x4_t *>(sw + woff[j][hh]);
        f32x4_t p[NBW][MBW];
#pragma unroll
        for (int qq = 0; qq < QW; ++qq) {
            bf16x8_t af[MBW];
#pragma unroll
            for (int b = 0; b < MBW; ++b)
                af[b] = *reinterpret_cast<const bf16x8_t *>(sa + aoff[b][qq]);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                bf16x8_t lo, hi;
                dequant16(wraw[j][qq >> 1], lo, hi);
                const bf16x8_t wb = (qq & 1) ? hi : lo;
#pragma unroll
                for (int b = 0; b < MBW; ++b)
                    p[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        wb, af[b], qq == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : p[j][b], 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int b = 0; b < MBW; ++b) {
                acc[j][b].x = __builtin_fmaf(s, p[j][b].x, acc[j][b].x);
                acc[j][b].y = __builtin_fmaf(s, p[j][b].y, acc[j][b].y);
                acc[j][b].z = __builtin_fmaf(s, p[j][b].z, acc[j][b].z);
                acc[j][b].w = __builtin_fmaf(s, p[j][b].w, acc[j][b].w);
            }
    }

    // ---- with KH == 2 the second group hands its sums to the first through
    // LDS (every wave has waited for all its loads: the last step waits for
    // none outstanding), and the first adds them: acc = group 0 + group 1.
    if constexpr (KH == 2) {
        f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);   // [4 waves][NBW][MBW][64]
        barrier_lds();
        if (computes && kh == 1) {
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int b = 0; b < MBW; ++b)
                    red[(((wave & 3u) * NBW + j) * MBW + b) * 64 + lane] = acc[j][b];
        }
        barrier_lds();
        if (!computes || kh == 1)
            return;
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int b = 0; b < MBW; ++b)
                acc[j][b] += red[((wave * NBW + j) * MBW + b) * 64 + lane];
    }

    if (!computes)
        return;
    // ---- epilogue: lane holds C[row][col..col+3] of each (j, b) tile.
    const uint32_t row_off = (MT / 2) * wm + rr;
    const uint32_t col_off = (NT / 2) * wn + 4u * gq;
    if (g.splits == 1) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int b = 0; b < MBW; ++b)
                store_c4(g, acc[j][b], m0 + row_off + 16u * b, n0 + col_off + 16u * j);
        return;
    }
    // Workspace [splits][m_tiles * MT][n_tiles * NT] FP32, whole tiles.
    const size_t ws_cols = (size_t)g.n_tiles * NT;
    float *wsp = g.ws + ((size_t)split * g.m_tiles * MT) * ws_cols;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MBW; ++b)
            *reinterpret_cast<f32x4_t *>(wsp + (size_t)(m0 + row_off + 16u * b) * ws_cols + n0 +
                                         col_off + 16u * j) = acc[j][b];
}

template <int MT, int NT, int WST, int AST, int KH, bool PROD, bool NTW>
hipError_t launch_tile_n(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if constexpr (!tile_variant_ok(MT / 16, NT / 16, WST, AST, 4 * KH + (PROD ? 2 : 0)) ||
                  !tile_depth_built(MT / 16, NT / 16, WST, AST)) {
        (void)g, (void)p, (void)stream;
        return hipErrorInvalidValue;
    } else {
    auto kern = w8a16_tile_kernel<MT, NT, WST, AST, KH, PROD, NTW>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), p.lds_bytes, kMaxLdsBytes,
                             lds_set);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g);
    e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1)
        return e;
    return launch_split_reduce(g, p.n_tiles * NT, p.m_tiles * MT, stream);
    }
}

template <int MT, int NT, int WST, int AST, int KH, bool PROD>
hipError_t launch_tile_t(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if (g.m_tiles == 1)
        return launch_tile_n<MT, NT, WST, AST, KH, PROD, true>(g, p, stream);
    return launch_tile_n<MT, NT, WST, AST, KH, PROD, false>(g, p, stream);
}

template <int MT, int NT, int WST, int AST>
hipError_t launch_tile_k(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.waves) {
    case 4: return launch_tile_t<MT, NT, WST, AST, 1, false>(g, p, stream);
    case 6: return launch_tile_t<MT, NT, WST, AST, 1, true>(g, p, stream);
    case 8: return launch_tile_t<MT, NT, WST, AST, 2, false>(g, p, stream);
    case 10: return launch_tile_t<MT, NT, WST, AST, 2, true>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Launch of the variant a (validated) plan names, for the tiles with
// m_blocks == MB; the table rows of other heights are compiled out.
template <uint32_t MB>
hipError_t launch_tile_rows(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    const uint32_t key = tile_variant_key(p.m_blocks, p.n_blocks, p.depth, p.a_depth);
#define W8A16_TILE_CASE(MB_, NB, D, AD)                                               \
    case tile_variant_key(MB_, NB, D, AD):                                            \
        if constexpr (MB_ == MB)                                                      \
            return launch_tile_k<16 * MB_, 16 * NB, D, AD>(g, p, stream);             \
        else                                                                          \
            return hipErrorInvalidValue;
    switch (key) {
    W8A16_TILE_VARIANTS(W8A16_TILE_CASE)
    default: return hipErrorInvalidValue;
    }
#undef W8A16_TILE_CASE
}

}  // namespace w8a16
