// Weight-streaming W8A16 GEMM kernel for small m (gfx950).
//
// Computes C = A * dequant(W)^T with one FP32 scale per 128x128 weight block
// applied once per 128-wide K step (page "w8a16_gemm_pipelined_m32.rs",
// doc comments of `w8a16_gemm_pipelined_m32_strided` and
// `W8A16_M32_K_BLOCK`; module doc, "Numerics").
//
// For m <= 64 the operation is bound by reading the FP8 weight from HBM, so
// the kernel is organised around streaming W once with 16-byte coalesced
// loads:
//
//   * A workgroup (W = 4, 8 or 16 waves) owns NBW 16-column blocks of C
//     (16 weight rows each) and MB 16-row blocks of C, over a range of
//     128-wide K steps.  Its waves take interleaved K steps (wave w: steps
//     s0+w, s0+w+W, ...), so at any time the W waves read W adjacent
//     128-byte pieces of each weight row.
//   * Per K step a wave loads its weight rows (8 lanes per 128-byte row
//     segment) and the A rows (16 lanes per 256-byte row segment) into
//     registers, writes them to its private LDS area in an XOR-swizzled
//     layout of 128-byte rows (A as two planes of half rows), and reads them
//     back in the 16x16x32 BF16 MFMA operand layout without bank conflicts.
//     The next step's loads are issued before the current step's math.
//   * The weight is the MFMA's first operand (its 16 rows are 16 columns of
//     C), A is the second; lane l then holds C[m = l%16][n = 4(l/16)..+3],
//     four adjacent outputs of one row.
//   * Inside a K step the MFMA's K index is a free relabelling of the 128
//     physical k: lane group g (= l/16) of MFMA q (0..3) covers physical k
//     32g+8q..32g+8q+7 in both operands.  That lets each lane read 32
//     contiguous weight bytes and 64 contiguous A bytes.
//   * FP8 -> BF16 with v_cvt_scalef32_pk_bf16_fp8 (scale 1.0): every E4M3
//     value, subnormals included, is a BF16 value, so the dequant is exact.
//   * Each workgroup starts its walk over its K range at a tile-dependent
//     offset and wraps around.  With a power-of-two K, workgroups that all
//     start at k = 0 send every concurrent request to the same few HBM
//     channels; rotated starts spread them.  The order of the scale-folded
//     step partials in each wave's accumulator changes; the set does not.
//   * Each step's 16x16 MFMA partial starts from zero and is folded into
//     the FP32 accumulator as acc = fma(scale, partial, acc).
//   * The waves' accumulators are added in LDS in wave order.  With K
//     split across workgroups (splits > 1), each split writes its FP32 tile
//     to a workspace, and the last workgroup to arrive at the tile's counter
//     adds the splits in split order, so every run gives the same bits.
//     Partials are published with agent-scope (write-through) stores and
//     read with agent-scope loads, with no L2 writeback.
//   * A plan with one row tile reads each weight byte once and loads it
//     with the non-temporal hint.
//   * Columns and rows past n and m are computed from clamped (valid)
//     addresses and never stored; A pitch padding is never read.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

using namespace dev;

constexpr uint32_t kW = 2048;   // LDS bytes of one 16-row weight block per K step
constexpr uint32_t kA = 4096;   // LDS bytes of one 16-row A block per K step

// Sum of the WAVES partial tiles of pair `pi` for one lane, in wave order.
// All LDS reads are issued before the additions.
template <int WAVES, int P>
__device__ __forceinline__ f32x4_t sum_waves(const f32x4_t *red, uint32_t pi, uint32_t lane)
{
    f32x4_t v[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        v[w] = red[(w * P + pi) * 64 + lane];
    f32x4_t s = v[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        s += v[w];
    return s;
}

// One workgroup's share of one GEMM: logical workgroup `lid` of g's grid
// (split lid % splits of tile lid / splits).  NTW: load the weight with the
// non-temporal hint (a plan with one row tile reads each weight byte once;
// with several row tiles the later reads should hit in the caches).
template <int MB, int NBW, int DEPTH, bool DIRECT, int WAVES, bool NTW>
__device__ __forceinline__ void stream_tile(const GemmArgs &g, uint32_t lid)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const uint32_t lane = threadIdx.x & 63u;
    // The wave index is the same for all lanes of a wave; saying so lets the
    // per-step scale loads be scalar loads.
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t split = lid % g.splits;
    const uint32_t tile = lid / g.splits;
    const uint32_t m_tile = tile % g.m_tiles;
    const uint32_t n_tile = tile / g.m_tiles;
    const uint32_t n0 = n_tile * (NBW * 16);
    const uint32_t m0 = m_tile * (MB * 16);
    const uint32_t ksteps = g.k / 128u;
    const uint32_t s0 = split * g.steps_per_split;
    const uint32_t s1 = min(ksteps, s0 + g.steps_per_split);
    // This wave's K steps: first, first + WAVES, ... (nw of them), each
    // mapped to physical step s0 + (i - s0 + rot) mod span.
    const uint32_t first = s0 + wave;
    const uint32_t nw = first < s1 ? (s1 - first + WAVES - 1) / WAVES : 0u;
    const uint32_t span = s1 - s0;
    const uint32_t rot = span ? (tile * kRotStride) % span : 0u;
    auto phys = [&](uint32_t i) {
        uint32_t x = i - s0 + rot;
        x = x >= span ? x - span : x;
        return s0 + x;
    };

    uint8_t *wl = lds + wave * (NBW * kW + (DIRECT ? 0u : MB * kA));
    uint8_t *al = wl + NBW * kW;

    // MFMA operand layout: row rr = lane%16 of a 16-row block, lane group
    // gq = lane/16 covers physical k 32gq..32gq+31 of the step.
    const uint32_t rr = lane & 15u, gq = lane >> 4;

    // ---- loop-invariant addressing -------------------------------------
    // DIRECT: each lane loads its own operand bytes (weight: 32 bytes of row
    // n0+16j+rr; A: 64 bytes of row m0+16b+rr).  Otherwise loads are
    // coalesced (weight row 16j+8h+lane/8, 16-byte chunk lane%8; A row
    // 16b+4q+lane/16, chunk lane%16) and go through the wave's LDS area.
    // Weight rows past n read the last valid row; A rows past m are zero.
    const uint8_t *wsrc[NBW][2];
    uint32_t wdst[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t r = 8u * h + (lane >> 3);
        wdst[h] = r * 128u + (((lane & 7u) ^ wswz(r)) * 16u);
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const uint32_t row = min(n0 + 16u * j + r, g.n - 1u);
            wsrc[j][h] = g.w + (size_t)row * g.k + (lane & 7u) * 16u;
        }
    }
    const uint8_t *asrc[MB][4];
    bool aok[MB][4];
    uint32_t adst[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t r = DIRECT ? rr : 4u * q + (lane >> 4);
        if (!DIRECT)
            adst[q] = ((lane & 15u) >> 3) * 2048u + r * 128u + (((lane & 7u) ^ wswz(r)) * 16u);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const uint32_t row = m0 + 16u * b + r;
            aok[b][q] = row < g.m;
            asrc[b][q] = g.a + (size_t)min(row, g.m - 1u) * g.a_stride * 2u +
                         (DIRECT ? (4u * gq + q) * 16u : (lane & 15u) * 16u);
        }
    }
    // LDS reads in MFMA layout (staged mode only).
    const uint32_t wrd0 = rr * 128u + (((2u * gq) ^ wswz(rr)) * 16u);
    const uint32_t wrd1 = rr * 128u + (((2u * gq + 1u) ^ wswz(rr)) * 16u);
    uint32_t ard[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        ard[q] = ((4u * gq + q) >> 3) * 2048u + rr * 128u + ((((4u * gq + q) & 7u) ^ wswz(rr)) * 16u);
    // Scale row of each weight block (a 16-row block never straddles two
    // 128-row scale blocks).
    const float *srow[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
        srow[j] = g.scale + (size_t)(min(n0 + 16u * j, g.n - 1u) / 128u) * ksteps;

    f32x4_t acc[NBW][MB];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Ring of DEPTH K steps in flight per wave.
    u32x4_t wr[DEPTH][NBW][2];
    u32x4_t ar[DEPTH][MB][4];
    float sr[DEPTH][NBW];

    auto issue = [&](int d, uint32_t t) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wr[d][j][h] = NTW ? __builtin_nontemporal_load(
                                        reinterpret_cast<const u32x4_t *>(wsrc[j][h] + t * 128u))
                                  : *reinterpret_cast<const u32x4_t *>(wsrc[j][h] + t * 128u);
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                ar[d][b][q] = aok[b][q]
                    ? *reinterpret_cast<const u32x4_t *>(asrc[b][q] + t * 256u)
                    : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            sr[d][j] = srow[j][t];
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if ((uint32_t)d < nw)
            issue(d, phys(first + WAVES * d));

    for (uint32_t base = 0; base < nw; base += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint32_t i = base + d;
            if (i >= nw)
                break;
            // Take step i out of the ring and refill the slot with step
            // i + DEPTH before doing step i's math.
            u32x4_t cw[NBW][2];
            u32x4_t ca[MB][4];
            float cs[NBW];
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                cw[j][0] = wr[d][j][0];
                cw[j][1] = wr[d][j][1];
                cs[j] = sr[d][j];
            }
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    ca[b][q] = ar[d][b][q];
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    *reinterpret_cast<u32x4_t *>(wl + j * kW + wdst[h]) = cw[j][h];
            if (!DIRECT) {
#pragma unroll
                for (int b = 0; b < MB; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<u32x4_t *>(al + b * kA + adst[q]) = ca[b][q];
            }
            if (i + DEPTH < nw)
                issue(d, phys(first + WAVES * (i + DEPTH)));

            bf16x8_t af[MB][4];
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    af[b][q] = DIRECT
                        ? __builtin_bit_cast(bf16x8_t, ca[b][q])
                        : *reinterpret_cast<const bf16x8_t *>(al + b * kA + ard[q]);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                const u32x4_t r0 = *reinterpret_cast<const u32x4_t *>(wl + j * kW + wrd0);
                const u32x4_t r1 = *reinterpret_cast<const u32x4_t *>(wl + j * kW + wrd1);
                bf16x8_t wb[4];
                dequant16(r0, wb[0], wb[1]);
                dequant16(r1, wb[2], wb[3]);
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[q], af[b][q], p, 0, 0, 0);
                    acc[j][b].x = __builtin_fmaf(cs[j], p.x, acc[j][b].x);
                    acc[j][b].y = __builtin_fmaf(cs[j], p.y, acc[j][b].y);
                    acc[j][b].z = __builtin_fmaf(cs[j], p.z, acc[j][b].z);
                    acc[j][b].w = __builtin_fmaf(cs[j], p.w, acc[j][b].w);
                }
            }
        }
    }

    // ---- add the 4 waves' partial sums in wave order ---------------------
    constexpr int P = NBW * MB;
    __syncthreads();
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            red[(wave * P + j * MB + b) * 64 + lane] = acc[j][b];
    __syncthreads();

    // Output position of a lane for pair (j, b).
    const uint32_t out_row_off = lane & 15u;
    const uint32_t out_col_off = 4u * (lane >> 4);

    if (g.splits == 1) {
        if constexpr (P < WAVES) {
            // Fewer output tiles than waves: spread the sums over all the
            // workgroup's threads, one output each (same wave order, so the
            // same bits), instead of leaving them to P waves (measured
            // 6.15 -> 5.87 us at 8 x 4096 x 4096, one tile of 16 waves).
            constexpr uint32_t F = P * 256u;   // floats per partial set
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
                // float f is component f % 4 of lane (f % 256) / 4 of tile f / 256
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
                const f32x4_t s = sum_waves<WAVES, P>(red, pi, lane);
                const uint32_t j = pi / MB, b = pi % MB;
                store_c4(g, s, m0 + 16u * b + out_row_off, n0 + 16u * j + out_col_off);
            }
        }
        return;
    }

    // ---- split-K: publish this split's tile, the last arrival adds all ----
    // Each split stores its FP32 partial tile with agent-scope atomic stores
    // (sc1: written through its XCD's L2) and waits until they have
    // completed before its arrival is counted.  The last split to arrive
    // reads every split's partial with agent-scope atomic loads (sc1: served
    // from the coherent copy, never from a stale line of its own L1 or L2)
    // issued after it has seen the count, and adds them in split order.
    // There is no fence: the partials are themselves the atomics, and a
    // release would write back (an acquire invalidate) the whole L2, each
    // measured as serialized over the grid (microseconds per call).  The
    // result does not depend on which XCD each split ran on.  The splits of
    // a tile are consecutive logical workgroups, which the logical id map
    // keeps on one XCD where the planner could arrange it.
    f32x4_t *ws_tile = reinterpret_cast<f32x4_t *>(g.ws) + (size_t)tile * g.splits * P * 64;
    for (uint32_t pi = wave; pi < (uint32_t)P; pi += WAVES)
        store_agent(ws_tile + ((size_t)split * P + pi) * 64 + lane,
                    sum_waves<WAVES, P>(red, pi, lane));
    wait_vm<0>();
    __syncthreads();
    __shared__ uint32_t last;
    uint32_t *counter = g.counters + (size_t)tile * kCounterStride;
    if (threadIdx.x == 0) {
        const uint32_t now = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) + 1u;
        last = now == g.splits ? 1u : 0u;
    }
    __syncthreads();
    if (!last)
        return;
    for (uint32_t pi = wave; pi < (uint32_t)P; pi += WAVES) {
        // eight partial loads in flight at a time (each is a round trip to
        // the coherent copy), added in split order
        f32x4_t s = load_agent(ws_tile + pi * 64 + lane);
        for (uint32_t sp = 1; sp < g.splits; sp += 8) {
            f32x4_t v[8];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u)
                if (sp + u < g.splits)
                    v[u] = load_agent(ws_tile + ((size_t)(sp + u) * P + pi) * 64 + lane);
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u)
                if (sp + u < g.splits)
                    s += v[u];
        }
        const uint32_t j = pi / MB, b = pi % MB;
        store_c4(g, s, m0 + 16u * b + out_row_off, n0 + 16u * j + out_col_off);
    }
    // ready for the next call that uses this workspace
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The weight is streamed with the non-temporal hint when the plan has one
// row tile (measured on MI355X, us per call: 8 x 4096 x 4096 6.00 -> 5.75,
// 16 x 12288 x 5120 15.0 -> 14.2, 1 x 1024 x 8192 5.58 -> 5.18; with two
// row tiles it cost 1-2 %: 32 x 6144 x 2048 6.80 -> 6.89).
// One instance per weight load form, chosen on the host (the batched grid,
// whose arms differ, chooses per arm in the kernel).
template <int MB, int NBW, int DEPTH, bool DIRECT, int WAVES, bool NTW>
__global__ __launch_bounds__(WAVES * 64) void w8a16_stream_kernel(GemmArgs g)
{
    stream_tile<MB, NBW, DEPTH, DIRECT, WAVES, NTW>(g, logical_wg(blockIdx.x, gridDim.x));
}

// Several independent GEMMs in one grid: problem i owns logical workgroups
// start[i] .. start[i + 1] - 1 (no K splits).  The problem is picked with
// wave-uniform selects, so its arguments stay in scalar registers.
template <int MB, int NBW, int DEPTH, bool DIRECT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void w8a16_stream_batched_kernel(BatchArgs b)
{
    const uint32_t lid = logical_wg(blockIdx.x, gridDim.x);
    GemmArgs g = b.g[0];
    uint32_t base = 0;
#pragma unroll
    for (uint32_t i = 1; i < W8A16_MAX_BATCH; ++i)
        if (i < b.count && lid >= b.start[i]) {
            g = b.g[i];
            base = b.start[i];
        }
    if (g.m_tiles == 1)
        stream_tile<MB, NBW, DEPTH, DIRECT, WAVES, true>(g, lid - base);
    else
        stream_tile<MB, NBW, DEPTH, DIRECT, WAVES, false>(g, lid - base);
}

template <int MB, int NBW, int DEPTH, bool DIRECT, int WAVES, bool NTW, typename Args>
hipError_t launch_stream_k(const Args &g, const w8a16_plan_t &p, hipStream_t stream)
{
    constexpr bool batched = std::is_same<Args, BatchArgs>::value;
    void (*kern)(Args);
    if constexpr (batched)
        kern = w8a16_stream_batched_kernel<MB, NBW, DEPTH, DIRECT, WAVES>;
    else
        kern = w8a16_stream_kernel<MB, NBW, DEPTH, DIRECT, WAVES, NTW>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), p.lds_bytes, kMaxLdsBytes,
                             lds_set);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g);
    return hipGetLastError();
}

template <int MB, int NBW, int DEPTH, bool DIRECT, int WAVES, typename Args>
hipError_t launch_stream_t(const Args &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if constexpr (std::is_same<Args, BatchArgs>::value)
        return launch_stream_k<MB, NBW, DEPTH, DIRECT, WAVES, false>(g, p, stream);
    else if (g.m_tiles == 1)
        return launch_stream_k<MB, NBW, DEPTH, DIRECT, WAVES, true>(g, p, stream);
    else
        return launch_stream_k<MB, NBW, DEPTH, DIRECT, WAVES, false>(g, p, stream);
}

template <int MB, int NBW, int DEPTH, bool DIRECT, typename Args>
hipError_t launch_stream_w(const Args &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.block / 64) {
    case 4: return launch_stream_t<MB, NBW, DEPTH, DIRECT, 4>(g, p, stream);
    case 8: return launch_stream_t<MB, NBW, DEPTH, DIRECT, 8>(g, p, stream);
    case 16: return launch_stream_t<MB, NBW, DEPTH, DIRECT, 16>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

// Batched launches are built for the default ring depth only (one K step
// per wave in flight, staged A), which is what their planner chooses.
template <int MB, int NBW, typename Args>
hipError_t launch_stream_mn(const Args &g, const w8a16_plan_t &p, hipStream_t stream)
{
    const bool direct = (p.flags & W8A16_FLAG_DIRECT) != 0;
    if constexpr (std::is_same<Args, BatchArgs>::value) {
        if (p.depth != 1 || direct)
            return hipErrorInvalidValue;
        return launch_stream_w<MB, NBW, 1, false>(g, p, stream);
    } else {
        switch (p.depth * 2 + (direct ? 1 : 0)) {
        case 2: return launch_stream_w<MB, NBW, 1, false>(g, p, stream);
        case 3: return launch_stream_w<MB, NBW, 1, true>(g, p, stream);
        case 4: return launch_stream_w<MB, NBW, 2, false>(g, p, stream);
        case 5: return launch_stream_w<MB, NBW, 2, true>(g, p, stream);
        case 8: return launch_stream_w<MB, NBW, 4, false>(g, p, stream);
        case 9: return launch_stream_w<MB, NBW, 4, true>(g, p, stream);
        default: return hipErrorInvalidValue;
        }
    }
}

template <typename Args>
hipError_t launch_stream_any(const Args &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.m_blocks * 100 + p.n_blocks) {
    case 101: return launch_stream_mn<1, 1>(g, p, stream);
    case 102: return launch_stream_mn<1, 2>(g, p, stream);
    case 103: return launch_stream_mn<1, 3>(g, p, stream);
    case 104: return launch_stream_mn<1, 4>(g, p, stream);
    case 108: return launch_stream_mn<1, 8>(g, p, stream);
    case 201: return launch_stream_mn<2, 1>(g, p, stream);
    case 202: return launch_stream_mn<2, 2>(g, p, stream);
    case 204: return launch_stream_mn<2, 4>(g, p, stream);
    case 208: return launch_stream_mn<2, 8>(g, p, stream);
    case 401: return launch_stream_mn<4, 1>(g, p, stream);
    case 402: return launch_stream_mn<4, 2>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_stream(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    return launch_stream_any(g, p, stream);
}

hipError_t launch_stream_batched(const BatchArgs &b, const w8a16_plan_t &p, hipStream_t stream)
{
    return launch_stream_any(b, p, stream);
}

}  // namespace w8a16
