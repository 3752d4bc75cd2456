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
//     into LDS with global_load_lds_dwordx4: the weight in a ring of WST
//     buffers (WST - 1 steps ahead, to cover HBM latency), A in two buffers
//     (one step ahead; it comes from L2).
//     Each lane picks the 16 bytes it moves so that the LDS image comes out
//     XOR-swizzled in 128-byte rows (conflict-free MFMA operand reads) while
//     every 8 lanes still read one whole 128-byte line.  The compiler does not track
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

constexpr uint32_t kTileM = 128;
constexpr uint32_t kABytes = kTileM * 256;   // one K step of A in LDS

// DMA one K step of A, or of the weight, of this wave's share into an LDS
// buffer.  __device__ functions rather than lambdas: a lambda in a kernel is
// also compiled for the host, where the DMA builtin does not exist.
template <int NA>
__device__ __forceinline__ void issue_a(uint8_t *dst, uint32_t wave, uint32_t t,
                                        const uint8_t *const *asrc)
{
#pragma unroll
    for (int u = 0; u < NA; ++u)
        __builtin_amdgcn_global_load_lds(asrc[u] + t * 256u,
                                         (lds_void_t *)(dst + (wave * NA + u) * 1024u), 16, 0, 0);
}

template <int NW>
__device__ __forceinline__ void issue_w(uint8_t *dst, uint32_t wave, uint32_t t,
                                        const uint8_t *const *wsrc)
{
#pragma unroll
    for (int u = 0; u < NW; ++u)
        __builtin_amdgcn_global_load_lds(wsrc[u] + t * 128u,
                                         (lds_void_t *)(dst + (wave * NW + u) * 1024u), 16, 0, 0);
}

template <int NT, int WST>
__global__ __launch_bounds__(256) void w8a16_tile_kernel(GemmArgs g)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr uint32_t kWBytes = NT * 128;
    constexpr int NA = kABytes / 1024 / 4;   // A DMA instructions per wave per step
    constexpr int NW = kWBytes / 1024 / 4;   // weight DMA instructions per wave per step
    // LDS: two A buffers, then WST weight buffers.
    uint8_t *const abuf = lds;
    uint8_t *const wbuf = lds + 2 * kABytes;
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
    // Logical step t of the split is physical step s0 + (t - s0 + rot) mod
    // span: tiles start their K walks at different offsets, which spreads
    // concurrent weight reads over the HBM channels for power-of-two K.
    const uint32_t span = s1 - s0;
    const uint32_t rot = span ? (tile * kRotStride) % span : 0u;
    auto phys = [&](uint32_t t) {
        uint32_t x = t - s0 + rot;
        x = x >= span ? x - span : x;
        return s0 + x;
    };

    // ---- DMA sources.  In LDS, A is two planes (K-step bytes 0..127 and
    // 128..255 of each row), each 128 rows x 128 bytes; the weight is NT rows
    // x 128 bytes.  Within a 128-byte row r, slot p holds 16-byte chunk
    // p ^ wswz(r % 16): with rows 128 bytes apart this makes the MFMA operand
    // reads below (16 lanes = 16 consecutive rows, one chunk each) free of
    // LDS bank conflicts on gfx950, which 256-byte rows are not.  A DMA
    // instruction fills 1 KiB of LDS = 8 rows of one plane; lane s writes
    // slot s % 8 of row s / 8, so it reads the chunk that slot holds.
    const uint8_t *asrc[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        const uint32_t i = wave * NA + u;          // 0..31: plane i / 16, rows 8(i % 16)..+7
        const uint32_t plane = i >> 4;
        const uint32_t r = 8u * (i & 15u) + (lane >> 3);
        const uint32_t c = 8u * plane + ((lane & 7u) ^ wswz(r & 15u));
        const uint32_t row = min(m0 + r, g.m - 1u);
        asrc[u] = g.a + (size_t)row * g.a_stride * 2u + c * 16u;
    }
    const uint8_t *wsrc[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        const uint32_t i = wave * NW + u;          // rows 8i..8i+7
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
            aoff[b][q] = ((4u * gq + q) >> 3) * (kTileM * 128u) + (64u * wm + 16u * b + rr) * 128u +
                         ((((4u * gq + q) & 7u) ^ wswz(rr)) * 16u);
    uint32_t woff[NBW][2];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            woff[j][h] = ((NT / 2) * wn + 16u * j + rr) * 128u +
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

    // Issue order, also in the prologue: iteration i issues A(i + 1), then
    // W(i + WST - 1).  The weight (from HBM) runs WST - 1 steps ahead, A (from
    // L2) one step ahead.
#pragma unroll
    for (int st = 0; st < WST - 2; ++st)
        if (s0 + st < s1)
            issue_w<NW>(wbuf + st * kWBytes, wave, phys(s0 + st), wsrc);
    if (s0 < s1)
        issue_a<NA>(abuf, wave, phys(s0), asrc);
    if (s0 + WST - 2 < s1)
        issue_w<NW>(wbuf + (WST - 2) * kWBytes, wave, phys(s0 + WST - 2), wsrc);

    for (uint32_t t = s0; t < s1; ++t) {
        const uint32_t idx = t - s0;
        // A(t) was issued one iteration ago, followed only by W(t + WST - 2)
        // (when that step exists); W(t) was issued before A(t).  So this
        // wave's DMA for step t is complete once at most that weight group is
        // outstanding.
        if (t + WST - 2 < s1)
            wait_vm<NW>();
        else
            wait_vm<0>();
        barrier_lds();
        if (t + 1 < s1)
            issue_a<NA>(abuf + ((idx + 1) & 1u) * kABytes, wave, phys(t + 1), asrc);
        if (t + WST - 1 < s1)
            issue_w<NW>(wbuf + ((idx + WST - 1) % WST) * kWBytes, wave, phys(t + WST - 1), wsrc);

        const uint8_t *sa = abuf + (idx & 1u) * kABytes;
        const uint8_t *sw = wbuf + (idx % WST) * kWBytes;
        const float s = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, svec), (int)(phys(t) - s0)));
        u32x4_t wraw[NBW][2];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wraw[j][h] = *reinterpret_cast<const u32x4_t *>(sw + woff[j][h]);
        f32x4_t p[NBW][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bf16x8_t af[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                af[b] = *reinterpret_cast<const bf16x8_t *>(sa + aoff[b][q]);
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

template <int NT, int WST>
hipError_t launch_tile_t(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    auto kern = w8a16_tile_kernel<NT, WST>;
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
    case 44: return launch_tile_t<64, 4>(g, p, stream);
    case 46: return launch_tile_t<64, 6>(g, p, stream);
    case 48: return launch_tile_t<64, 8>(g, p, stream);
    case 83: return launch_tile_t<128, 3>(g, p, stream);
    case 84: return launch_tile_t<128, 4>(g, p, stream);
    case 85: return launch_tile_t<128, 5>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w8a16
