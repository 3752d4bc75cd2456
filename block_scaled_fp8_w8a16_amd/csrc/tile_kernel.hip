// Tiled W8A16 GEMM kernel for large m (gfx950), plus the fixed-order
// reduction of its K splits.
//
// Same operation as the stream kernel (page "w8a16_gemm_pipelined_m32.rs":
// operand layouts in the doc comment of `w8a16_gemm_pipelined_m32_strided`,
// one FP32 scale per 128x128 weight block folded once per 128-wide K step,
// `W8A16_M32_K_BLOCK`).  The page's large-row path is a 128-row tile that
// shares the dequantized weight across all its rows
// (`w8a16_gemm_pipelined_by_m`); this is that idea rebuilt for MI355X:
//
//   * A workgroup (4 waves, 2 x 2) owns a 128-row x NT-column tile of C over
//     a range of 128-wide K steps.  Each wave owns 64 rows x NT/2 columns:
//     4 x NT/32 MFMA 16x16x32 tiles.
//   * Per K step the workgroup stages A (128 rows x 256 bytes of BF16) and
//     the weight (NT rows x 128 bytes of FP8) straight from global memory
//     into LDS with global_load_lds_dwordx4, in a ring of STAGES buffers.
//     Each lane picks the 16 bytes it moves so that the LDS image comes out
//     XOR-swizzled (conflict-free MFMA operand reads) while every group of
//     lanes still reads whole 128-byte lines.  The compiler does not track
//     these DMA writes, so the kernel waits for them itself (s_waitcnt
//     vmcnt) and a workgroup barrier per step publishes them and retires
//     the buffer being refilled.
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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace w8a16 {

namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr uint32_t kTileM = 128;
constexpr uint32_t kABytes = kTileM * 256;   // one K step of A in LDS

// s_waitcnt vmcnt(N) with lgkmcnt and expcnt left alone.  The memory clobber
// keeps LDS reads of the DMA'd data from moving above the wait.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that does not drain outstanding global loads (the
// ordinary __syncthreads() waits for every in-flight DMA step): it waits only
// for this wave's LDS reads, so no wave can refill a buffer another wave is
// still reading.  The DMA data of a step is covered by wait_vm() before it.
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// DMA one K step (A and weight) of this wave's share into LDS stage buffer
// `sb`.  A __device__ function rather than a lambda: a lambda in a kernel is
// also compiled for the host, where the DMA builtin does not exist.
template <int NA, int NW>
__device__ __forceinline__ void issue_step(uint8_t *sb, uint32_t wave, uint32_t t,
                                           const uint8_t *const *asrc,
                                           const uint8_t *const *wsrc)
{
#pragma unroll
    for (int u = 0; u < NA; ++u)
        __builtin_amdgcn_global_load_lds(asrc[u] + t * 256u,
                                         (lds_void_t *)(sb + (wave * NA + u) * 1024u), 16, 0, 0);
#pragma unroll
    for (int u = 0; u < NW; ++u)
        __builtin_amdgcn_global_load_lds(wsrc[u] + t * 128u,
                                         (lds_void_t *)(sb + kABytes + (wave * NW + u) * 1024u),
                                         16, 0, 0);
}

template <int NT, int STAGES>
__global__ __launch_bounds__(256) void w8a16_tile_kernel(GemmArgs g)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr uint32_t kWBytes = NT * 128;
    constexpr uint32_t kStage = kABytes + kWBytes;
    constexpr int NA = kABytes / 1024 / 4;   // A DMA instructions per wave per step
    constexpr int NW = kWBytes / 1024 / 4;   // weight DMA instructions per wave per step
    constexpr int PER_STEP = NA + NW;
    constexpr int NBW = NT / 32;             // 16-column blocks per wave
    static_assert(NW >= 1 && NBW >= 1, "tile too small");

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave & 1u, wn = wave >> 1;
    const uint32_t lid = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t split = lid % g.splits;
    const uint32_t tile = lid / g.splits;
    const uint32_t m_tile = tile % g.m_tiles;
    const uint32_t n_tile = tile / g.m_tiles;
    const uint32_t m0 = m_tile * kTileM;
    const uint32_t n0 = n_tile * NT;
    const uint32_t ksteps = g.k / 128u;
    const uint32_t s0 = split * g.steps_per_split;
    const uint32_t s1 = min(ksteps, s0 + g.steps_per_split);

    // ---- DMA sources: lane s of A instruction i fills LDS slot s of rows
    // 4i..4i+3 (16 slots of 16 bytes per 256-byte row); slot p of row r holds
    // chunk p ^ (r % 16).  Weight instruction i covers rows 8i..8i+7 (8 slots
    // per 128-byte row); slot p of row r holds chunk p ^ wswz(r % 16).
    const uint8_t *asrc[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        const uint32_t i = wave * NA + u;
        const uint32_t r = 4u * i + (lane >> 4);
        const uint32_t c = (lane & 15u) ^ (r & 15u);
        const uint32_t row = min(m0 + r, g.m - 1u);
        asrc[u] = g.a + (size_t)row * g.a_stride * 2u + c * 16u;
    }
    const uint8_t *wsrc[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        const uint32_t i = wave * NW + u;
        const uint32_t r = 8u * i + (lane >> 3);
        const uint32_t c = (lane & 7u) ^ wswz(r & 15u);
        const uint32_t row = min(n0 + r, g.n - 1u);
        wsrc[u] = g.w + (size_t)row * g.k + c * 16u;
    }
    // ---- MFMA operand reads: row rr = lane % 16 of a 16-row block, lane
    // group gq = lane / 16 covers physical k 32gq..32gq+31 of the step (MFMA
    // q takes k 32gq+8q..+7 from both operands).
    const uint32_t rr = lane & 15u, gq = lane >> 4;
    uint32_t aoff[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            aoff[b][q] = (64u * wm + 16u * b + rr) * 256u + (((4u * gq + q) ^ rr) * 16u);
    uint32_t woff[NBW][2];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            woff[j][h] = kABytes + ((NT / 2) * wn + 16u * j + rr) * 128u +
                         (((2u * gq + h) ^ wswz(rr)) * 16u);
    // Scales of the tile's 128-row block for this split's steps (at most 64,
    // which the planner guarantees), one per lane: lane l holds step s0 + l.
    // They are loaded and waited for before any DMA is issued, so the loop
    // has no vector loads of its own; each step reads its scale with readlane.
    const float *srow = g.scale + (size_t)(min(n0, g.n - 1u) / 128u) * ksteps;
    const float svec = (s0 + lane < s1) ? srow[s0 + lane] : 0.f;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt untouched

    f32x4_t acc[NBW][4];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (s0 + st < s1)
            issue_step<NA, NW>(lds + st * kStage, wave, s0 + st, asrc, wsrc);

    for (uint32_t t = s0; t < s1; ++t) {
        const uint32_t idx = t - s0;
        // This wave's DMA for step t is done once at most the later steps'
        // groups (up to STAGES-2 of them) are still outstanding.
        const uint32_t later = min((uint32_t)(STAGES - 2), s1 - 1u - t);
        if (STAGES >= 3 && later >= 1) {
            if (STAGES >= 4 && later >= 2)
                wait_vm<(STAGES >= 4 ? 2 : 0) * PER_STEP>();
            else
                wait_vm<(STAGES >= 3 ? 1 : 0) * PER_STEP>();
        } else {
            wait_vm<0>();
        }
        barrier_lds();
        if (t + STAGES - 1 < s1)
            issue_step<NA, NW>(lds + ((idx + STAGES - 1) % STAGES) * kStage, wave,
                               t + STAGES - 1, asrc, wsrc);

        const uint8_t *sb = lds + (idx % STAGES) * kStage;
        const float s = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, svec), (int)idx));
        u32x4_t wraw[NBW][2];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wraw[j][h] = *reinterpret_cast<const u32x4_t *>(sb + woff[j][h]);
        f32x4_t p[NBW][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bf16x8_t af[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                af[b] = *reinterpret_cast<const bf16x8_t *>(sb + aoff[b][q]);
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                bf16x8_t lo, hi;
                dequant16(wraw[j][q >> 1], lo, hi);
                const bf16x8_t wb = (q & 1) ? hi : lo;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    p[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        wb, af[b], q == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : p[j][b], 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                acc[j][b].x = __builtin_fmaf(s, p[j][b].x, acc[j][b].x);
                acc[j][b].y = __builtin_fmaf(s, p[j][b].y, acc[j][b].y);
                acc[j][b].z = __builtin_fmaf(s, p[j][b].z, acc[j][b].z);
                acc[j][b].w = __builtin_fmaf(s, p[j][b].w, acc[j][b].w);
            }
    }

    // ---- epilogue: lane holds C[row][col..col+3] of each (j, b) tile.
    const uint32_t row_off = 64u * wm + rr;
    const uint32_t col_off = (NT / 2) * wn + 4u * gq;
    if (g.splits == 1) {
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                store_c4(g, acc[j][b], m0 + row_off + 16u * b, n0 + col_off + 16u * j);
        return;
    }
    // Workspace [splits][m_tiles * 128][n_tiles * NT] FP32, whole tiles.
    const size_t ws_cols = (size_t)g.n_tiles * NT;
    float *wsp = g.ws + ((size_t)split * g.m_tiles * kTileM) * ws_cols;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            *reinterpret_cast<f32x4_t *>(wsp + (size_t)(m0 + row_off + 16u * b) * ws_cols + n0 +
                                         col_off + 16u * j) = acc[j][b];
}

// C = sum over splits, in split order, of the workspace tiles; one thread
// per 4 adjacent outputs.
__global__ __launch_bounds__(256) void w8a16_split_reduce_kernel(GemmArgs g, uint32_t ws_cols,
                                                                 uint32_t ws_rows)
{
    const uint32_t quads = ws_cols / 4u;
    const uint64_t id = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t row = (uint32_t)(id / quads);
    const uint32_t col = (uint32_t)(id % quads) * 4u;
    if (row >= g.m || col >= g.n)
        return;
    const size_t plane = (size_t)ws_rows * ws_cols;
    const float *p = g.ws + (size_t)row * ws_cols + col;
    f32x4_t s = *reinterpret_cast<const f32x4_t *>(p);
    for (uint32_t sp = 1; sp < g.splits; ++sp)
        s += *reinterpret_cast<const f32x4_t *>(p + sp * plane);
    store_c4(g, s, row, col);
}

template <int NT, int STAGES>
hipError_t launch_tile_t(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    auto kern = w8a16_tile_kernel<NT, STAGES>;
    static bool attr_set = false;
    if (p.lds_bytes > 65536 && !attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)p.lds_bytes);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1)
        return e;
    const uint32_t ws_cols = p.n_tiles * NT;
    const uint32_t ws_rows = p.m_tiles * kTileM;
    const uint64_t threads = (uint64_t)g.m * (ws_cols / 4u);
    const uint32_t blocks = (uint32_t)((threads + 255u) / 256u);
    hipLaunchKernelGGL(w8a16_split_reduce_kernel, dim3(blocks), dim3(256), 0, stream, g, ws_cols,
                       ws_rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tile(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.n_blocks * 10 + p.depth) {
    case 42: return launch_tile_t<64, 2>(g, p, stream);
    case 43: return launch_tile_t<64, 3>(g, p, stream);
    case 82: return launch_tile_t<128, 2>(g, p, stream);
    case 83: return launch_tile_t<128, 3>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w8a16
