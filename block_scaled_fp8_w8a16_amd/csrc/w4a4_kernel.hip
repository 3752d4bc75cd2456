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
//   * K is walked in groups of 4 steps: a lane's scale bytes for 4 steps of
//     one row are 16 contiguous bytes, one load per group (one dword per
//     step when K is not a multiple of 512).
//   * Tiled kernel: a workgroup owns NBW 16-column blocks of C and MB 16-row
//     blocks over all of K; its waves take interleaved groups, the next
//     group's loads in flight while one is computed; every A fragment feeds
//     the NBW weight blocks from registers; rows of A past m are not loaded.
//     The waves' partial tiles are added in LDS in wave order, then stored
//     as BF16.
//   * Persistent kernel (9..32 rows over a wide weight): one workgroup per
//     CU stages all of A and its scales in LDS once; then each wave walks
//     its own 16-row weight tiles over all of K, taking A from LDS.  A is
//     read once per CU instead of once per tile.  Tiles are dealt out
//     round-robin (they all cost the same), so there is no tile counter.
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

// Every global load of these kernels is a raw buffer load (make_rsrc,
// load16, load4): steps past K, rows past m or n and the prefetch past a
// wave's last group are offsets past the resource, which read zeros, so no
// load sits under a branch and the compiler's wait counts stay exact.

// Scale dwords of the 4 K steps of group `gidx` for one row (`row_off` =
// the row's first scale byte in the resource): dword e holds the 4 block
// scales of step 4 gidx + e.  SC16 (K a multiple of 512, every group
// whole): one 16-byte load.  Otherwise one dword per step.  Steps at or
// past `ksteps` read zeros.
template <bool SC16>
__device__ __forceinline__ void load_scales(uint32_t (&d)[4], __amdgpu_buffer_rsrc_t r,
                                            uint32_t row_off, uint32_t gidx, uint32_t ksteps)
{
    if constexpr (SC16) {
        const u32x4_t v = load16<false>(r, row_off + (4u * gidx < ksteps ? 16u * gidx : kOob));
        d[0] = v.x;
        d[1] = v.y;
        d[2] = v.z;
        d[3] = v.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t t = 4u * gidx + e;
            d[e] = load4(r, row_off + (t < ksteps ? 4u * t : kOob));
        }
    }
}

// Byte offset of step t inside a row (16 gq added per lane), or past the
// resource for a step at or past ksteps.
__device__ __forceinline__ uint32_t step_off(uint32_t t, uint32_t ksteps)
{
    return t < ksteps ? 64u * t : kOob;
}

// The byte of lane group gq (its 32-element block) of a step's scale dword.
__device__ __forceinline__ uint32_t scale_byte(uint32_t d, uint32_t gq)
{
    return (d >> (8u * gq)) & 0xffu;
}

// One group of 4 K steps of a wave: weight and A fragments and scales.
template <int MB, int NBW>
struct MxGroup {
    u32x4_t w[4][NBW];
    u32x4_t a[4][MB];
    uint32_t ws[NBW][4];
    uint32_t as[MB][4];
};

// Groups of 4 K steps in flight per wave (the one being computed included).
constexpr int kTileBufs = 2;
constexpr int kPsBufs = 3;
// Persistent kernel: A chunks (16 bytes) and scale dwords staged per
// thread and batch.
constexpr uint32_t kStageA = 4;
constexpr uint32_t kStageS = 2;

template <int MB, int NBW, int WAVES, bool NTW, bool SC16>
__global__ __launch_bounds__(WAVES * 64) void w8a16_w4a4_kernel(MxArgs g)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tile = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t m0 = (tile % g.m_tiles) * (MB * 16);
    const uint32_t n0 = (tile / g.m_tiles) * (NBW * 16);
    const uint32_t ksteps = g.k / 128u;
    const uint32_t kb = g.k / 32u;                     // scale bytes per row
    const uint32_t groups = (ksteps + 3u) / 4u;
    const uint32_t rr = lane & 15u, gq = lane >> 4;
    // this wave's groups of 4 K steps: wave, wave + WAVES, ... (ng of them),
    // walked from a per-tile rotation so that neighbouring tiles read
    // different K; index ng and above stand for "no group" (zeros)
    const uint32_t ng = wave < groups ? (groups - wave + WAVES - 1) / WAVES : 0u;
    const uint32_t rot = (tile * kRotStride) % groups;
    auto gphys = [&](uint32_t i) {
        if (i >= ng)
            return groups;
        const uint32_t x = wave + WAVES * i + rot;
        return x >= groups ? x - groups : x;
    };

    // resources over the tile's rows; lane offsets: row rr of each 16-row
    // block, byte 16 gq of a step's 64 bytes
    const uint32_t wrows = min((uint32_t)NBW * 16u, g.n - n0);
    const uint32_t arows = min((uint32_t)MB * 16u, g.m - m0);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(g.w + (size_t)n0 * (g.k / 2u), wrows * (g.k / 2u));
    const __amdgpu_buffer_rsrc_t wsr = make_rsrc(g.w_scale + (size_t)n0 * kb, wrows * kb);
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(g.a + (size_t)m0 * g.a_stride, arows * g.a_stride);
    const __amdgpu_buffer_rsrc_t asr = make_rsrc(g.a_scale + (size_t)m0 * kb, arows * kb);
    uint32_t wo[NBW], wso[NBW], ao[MB], aso[MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        wo[j] = (16u * j + rr) * (g.k / 2u) + 16u * gq;
        wso[j] = (16u * j + rr) * kb;
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        ao[b] = (16u * b + rr) * g.a_stride + 16u * gq;
        aso[b] = (16u * b + rr) * kb;
    }

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](MxGroup<MB, NBW> &q, uint32_t gidx) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t so = step_off(4u * gidx + e, ksteps);
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                q.w[e][j] = load16<NTW>(wr, wo[j] + so);
#pragma unroll
            for (int b = 0; b < MB; ++b)
                q.a[e][b] = load16<false>(ar, ao[b] + so);
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            load_scales<SC16>(q.ws[j], wsr, wso[j], gidx, ksteps);
#pragma unroll
        for (int b = 0; b < MB; ++b)
            load_scales<SC16>(q.as[b], asr, aso[b], gidx, ksteps);
    };
    // steps past K hold zero data and zero scale bytes (2^-127): they add 0
    auto compute = [&](const MxGroup<MB, NBW> &q) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    acc[j][b] = mx_step(q.w[e][j], scale_byte(q.ws[j][e], gq), q.a[e][b],
                                        scale_byte(q.as[b][e], gq), acc[j][b]);
    };
    // a straight-line ring: every slot issues and computes (a group past
    // the wave's last reads zeros and adds 0), so no load sits under a
    // branch; the scheduling barrier keeps each prefetch ahead of the
    // compute that follows it
    MxGroup<MB, NBW> buf[kTileBufs];
#pragma unroll
    for (int s = 0; s < kTileBufs - 1; ++s)
        issue(buf[s], gphys(s));
    for (uint32_t i = 0; i < ng; i += kTileBufs) {
#pragma unroll
        for (int s = 0; s < kTileBufs; ++s) {
            issue(buf[(s + kTileBufs - 1) % kTileBufs], gphys(i + s + kTileBufs - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(buf[s]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    reduce_store<MB, NBW, WAVES>(g, acc, m0, n0, wave, lane);
}

// Persistent kernel.  Workgroup g owns the contiguous 16-row weight tiles
// [g n16 / G, (g + 1) n16 / G) and all of their K: items (tile, group of 4
// K steps), tile-major, split into WAVES equal contiguous ranges, one per
// wave.  A (MB 16-row blocks, all of K, rows padded by 16 bytes) and its
// scale bytes are staged in LDS once; each wave then streams its weight
// items with kPsBufs groups in flight.  A wave that covers a whole
// tile stores it; a tile split between waves leaves one partial per wave
// in LDS (slot 0 for the wave's first tile, slot 1 for its last), and the
// wave holding the tile's first item adds them in wave order.
template <int MB, int WAVES, bool SC16>
__global__ __launch_bounds__(WAVES * 64) void w8a16_w4a4_ps_kernel(MxArgs g)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ksteps = g.k / 128u;
    const uint32_t kb = g.k / 32u;                     // scale bytes per row
    const uint32_t groups = (ksteps + 3u) / 4u;
    const uint32_t cpr = g.k / 32u;                    // 16-byte chunks per row
    const uint32_t pitch = 16u * (cpr + 1u);           // LDS row pitch of A (bytes)
    const uint32_t abytes = w4a4_ps_a_bytes(MB, g.k);
    const uint32_t sbytes = w4a4_ps_s_bytes(MB, g.k);
    uint8_t *alds = lds;                               // [MB * 16][pitch]
    uint8_t *slds = lds + abytes;                      // [MB * 16][kb]
    f32x4_t *part = reinterpret_cast<f32x4_t *>(lds + abytes + sbytes);  // [WAVES][2][MB][64]
    const uint32_t rr = lane & 15u, gq = lane >> 4;

    // tiles and items of this workgroup and wave
    const uint32_t t_lo = blockIdx.x * g.tiles_base + min(blockIdx.x, g.tiles_extra);
    const uint32_t items = (g.tiles_base + (blockIdx.x < g.tiles_extra ? 1u : 0u)) * groups;
    auto range_start = [&](uint32_t w) { return (uint32_t)((uint64_t)w * items / WAVES); };
    const uint32_t s = range_start(wave), e = range_start(wave + 1u);

    // 1. A and its scales into LDS through registers, in batches of kStageA
    // 16-byte chunks and kStageS scale dwords per thread.  Thread x copies
    // row x % R (R = 16 MB rows) of A, chunks x / R + j (threads / R) of
    // the row; rows past m read zeros.  The last batch's loads are issued
    // before the weight ring's first groups and written to LDS after them,
    // so the ring is in flight while A arrives.
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(g.a, g.m * g.a_stride);
    const __amdgpu_buffer_rsrc_t asr = make_rsrc(g.a_scale, g.m * kb);
    constexpr uint32_t kThreads = WAVES * 64u;
    constexpr uint32_t kRows = MB * 16u;
    constexpr uint32_t kColStep = kThreads / kRows;    // chunk step of one thread
    const uint32_t arow = threadIdx.x % kRows, acol = threadIdx.x / kRows;
    const uint32_t sdwords = sbytes / 4u;
    const uint32_t a_batches = (cpr + kStageA * kColStep - 1u) / (kStageA * kColStep);
    const uint32_t s_batches = (sdwords + kStageS * kThreads - 1u) / (kStageS * kThreads);
    const uint32_t batches = max(a_batches, s_batches);
    u32x4_t av[kStageA];
    uint32_t sv[kStageS];
    auto stage_load = [&](uint32_t bi) {
#pragma unroll
        for (uint32_t c = 0; c < kStageA; ++c) {
            const uint32_t ch = acol + (bi * kStageA + c) * kColStep;
            av[c] = load16<false>(ar, ch < cpr ? arow * g.a_stride + 16u * ch : kOob);
        }
#pragma unroll
        for (uint32_t c = 0; c < kStageS; ++c) {
            const uint32_t q = (bi * kStageS + c) * kThreads + threadIdx.x;
            sv[c] = load4(asr, q < sdwords ? 4u * q : kOob);
        }
    };
    auto stage_store = [&](uint32_t bi) {
#pragma unroll
        for (uint32_t c = 0; c < kStageA; ++c) {
            const uint32_t ch = acol + (bi * kStageA + c) * kColStep;
            if (ch < cpr)
                *reinterpret_cast<u32x4_t *>(alds + arow * pitch + 16u * ch) = av[c];
        }
#pragma unroll
        for (uint32_t c = 0; c < kStageS; ++c) {
            const uint32_t q = (bi * kStageS + c) * kThreads + threadIdx.x;
            if (q < sdwords)
                *reinterpret_cast<uint32_t *>(slds + 4u * q) = sv[c];
        }
    };
    for (uint32_t bi = 0; bi + 1u < batches; ++bi) {
        stage_load(bi);
        stage_store(bi);
    }
    stage_load(batches - 1u);
    __builtin_amdgcn_sched_barrier(0);

    // 2. the weight ring's first groups (buffer loads into registers)
    const uint32_t wo = rr * (g.k / 2u) + 16u * gq;   // lane offset inside a tile
    const uint32_t wso = rr * kb;
    struct Group {
        u32x4_t w[4];
        uint32_t ws[4];
    };
    // (tile, group) cursors of the next item to issue and to compute:
    // items are walked in order, so no division per item
    uint32_t itl = s / groups, igx = s % groups;
    uint32_t ctl = itl, cgx = igx;
    auto issue = [&](Group &q, uint32_t i) {
        const bool ok = i < e;
        const uint32_t tl = ok ? itl : 0u;
        const uint32_t gidx = ok ? igx : groups;
        if (++igx == groups) {
            igx = 0;
            ++itl;
        }
        const uint32_t t = t_lo + tl;
        const uint32_t rows = min(16u, g.n - 16u * t);
        const __amdgpu_buffer_rsrc_t wr =
            make_rsrc(g.w + (size_t)(16u * t) * (g.k / 2u), rows * (g.k / 2u));
        const __amdgpu_buffer_rsrc_t wsr = make_rsrc(g.w_scale + (size_t)(16u * t) * kb, rows * kb);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            q.w[e4] = load16<true>(wr, wo + step_off(4u * gidx + e4, ksteps));
        load_scales<SC16>(q.ws, wsr, wso, gidx, ksteps);
    };
    Group buf[kPsBufs];
#pragma unroll
    for (int b = 0; b < kPsBufs - 1; ++b)
        issue(buf[b], s + b);
    __builtin_amdgcn_sched_barrier(0);
    stage_store(batches - 1u);
    barrier_lds();

    // 3. the wave's items; a tile ends at its last group or the range's end
    const uint32_t t_first = s / groups;
    f32x4_t acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto store_tile = [&](const f32x4_t (&v)[MB], uint32_t tl) {
        // lane l holds C[row l % 16 of block b][n0 + 4 (l / 16) .. +3]
        const uint32_t col = 16u * (t_lo + tl) + 4u * gq;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const uint32_t row = 16u * b + rr;
            if (row < g.m) {
                uint16_t *dst = reinterpret_cast<uint16_t *>(g.c) + (size_t)row * g.c_stride + col;
                const float x[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    if (col + e4 < g.n)
                        dst[e4] = (uint16_t)f32_to_bf16_bits(x[e4]);
            }
        }
    };
    auto compute = [&](const Group &q, uint32_t i) {
        const uint32_t tl = ctl, gidx = cgx;
        if (++cgx == groups) {
            cgx = 0;
            ++ctl;
        }
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const uint32_t t = 4u * gidx + e4;
            const uint32_t tk = t < ksteps ? t : 0u;   // past K: zero weight, any A
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const uint32_t r = 16u * b + rr;
                const u32x4_t a = *reinterpret_cast<const u32x4_t *>(alds + r * pitch +
                                                                     64u * tk + 16u * gq);
                const uint32_t as = *reinterpret_cast<const uint32_t *>(slds + r * kb + 4u * tk);
                acc[b] = mx_step(q.w[e4], scale_byte(q.ws[e4], gq), a, scale_byte(as, gq), acc[b]);
            }
        }
        if (gidx == groups - 1u || i == e - 1u) {
            if (tl * groups >= s && (tl + 1u) * groups <= e) {
                store_tile(acc, tl);
            } else {
                const uint32_t slot = tl == t_first ? 0u : 1u;
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    part[((wave * 2u + slot) * MB + b) * 64u + lane] = acc[b];
            }
#pragma unroll
            for (int b = 0; b < MB; ++b)
                acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    for (uint32_t i = s; i < e; i += kPsBufs) {
#pragma unroll
        for (int b = 0; b < kPsBufs; ++b) {
            issue(buf[(b + kPsBufs - 1) % kPsBufs], i + b + kPsBufs - 1);
            __builtin_amdgcn_sched_barrier(0);
            if (i + b < e)
                compute(buf[b], i + b);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();

    // 4. split tiles: the wave whose range holds a tile's first item but not
    // its last (that tile is the wave's last) adds its own partial and the
    // slot-0 partials of the following waves that start inside the tile
    if (e > s) {
        const uint32_t tl = (e - 1u) / groups;
        if (tl * groups >= s && (tl + 1u) * groups > e) {
            const uint32_t slot = tl == t_first ? 0u : 1u;
            f32x4_t sum[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b)
                sum[b] = part[((wave * 2u + slot) * MB + b) * 64u + lane];
            for (uint32_t w = wave + 1u; w < (uint32_t)WAVES; ++w) {
                const uint32_t ws0 = range_start(w), we0 = range_start(w + 1u);
                if (ws0 >= (tl + 1u) * groups)
                    break;
                if (we0 > ws0) {
#pragma unroll
                    for (int b = 0; b < MB; ++b)
                        sum[b] += part[((w * 2u) * MB + b) * 64u + lane];
                }
            }
            store_tile(sum, tl);
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

template <int MB, int NBW, bool NTW, bool SC16>
hipError_t launch_w4a4_v(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    static std::atomic<uint64_t> lds_set[3];
    switch (p.waves) {
    case 4:
        return launch_mx(w8a16_w4a4_kernel<MB, NBW, 4, NTW, SC16>, g, p, stream, lds_set[0]);
    case 8:
        if constexpr (w4a4_variant_ok(MB, NBW, 8))
            return launch_mx(w8a16_w4a4_kernel<MB, NBW, 8, NTW, SC16>, g, p, stream, lds_set[1]);
        break;
    case 16:
        if constexpr (w4a4_variant_ok(MB, NBW, 16))
            return launch_mx(w8a16_w4a4_kernel<MB, NBW, 16, NTW, SC16>, g, p, stream, lds_set[2]);
        break;
    default: break;
    }
    return hipErrorInvalidValue;
}

// Nontemporal weight loads when no other row tile reads the same weight;
// 16-byte scale loads when every group of 4 K steps is whole.
template <int MB, int NBW>
hipError_t launch_w4a4_mn(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    const bool sc16 = g.k % 512u == 0;
    if (g.m_tiles == 1)
        return sc16 ? launch_w4a4_v<MB, NBW, true, true>(g, p, stream)
                    : launch_w4a4_v<MB, NBW, true, false>(g, p, stream);
    return sc16 ? launch_w4a4_v<MB, NBW, false, true>(g, p, stream)
                : launch_w4a4_v<MB, NBW, false, false>(g, p, stream);
}

template <int MB, bool SC16>
hipError_t launch_w4a4_ps_v(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    static std::atomic<uint64_t> lds_set[3];
    switch (p.waves) {
    case 4: return launch_mx(w8a16_w4a4_ps_kernel<MB, 4, SC16>, g, p, stream, lds_set[0]);
    case 8: return launch_mx(w8a16_w4a4_ps_kernel<MB, 8, SC16>, g, p, stream, lds_set[1]);
    case 16: return launch_mx(w8a16_w4a4_ps_kernel<MB, 16, SC16>, g, p, stream, lds_set[2]);
    default: return hipErrorInvalidValue;
    }
}

template <int MB>
hipError_t launch_w4a4_ps_m(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    return g.k % 512u == 0 ? launch_w4a4_ps_v<MB, true>(g, p, stream)
                           : launch_w4a4_ps_v<MB, false>(g, p, stream);
}

}  // namespace

hipError_t launch_w4a4(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if (p.kernel == W8A16_KERNEL_W4A4_PS) {
        switch (p.m_blocks) {
        case 1: return launch_w4a4_ps_m<1>(g, p, stream);
        case 2: return launch_w4a4_ps_m<2>(g, p, stream);
        case 4: return launch_w4a4_ps_m<4>(g, p, stream);
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
