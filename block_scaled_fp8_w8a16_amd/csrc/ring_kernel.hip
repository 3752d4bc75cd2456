// Ring kernel: weight-streaming W8A16 GEMM for small m with a deep ring of
// LDS-DMA stages (gfx950).
//
// Same operation as the other kernels (page "w8a16_gemm_pipelined_m32.rs":
// operand layouts in the doc comment of `w8a16_gemm_pipelined_m32_strided`,
// one FP32 scale per 128x128 weight block folded once per 128-wide K step,
// `W8A16_M32_K_BLOCK`).  For m <= 64 the cost is reading the FP8 weight
// once; this kernel is shaped by what gets that read close to HBM speed on
// MI355X:
//
//   * A workgroup (8 or 16 waves) owns NBW 16-column blocks and MB 16-row
//     blocks of C over all of K.  K is cut into stages of SK steps and a
//     ring of NST stages is in flight (with K = 4096 and 16 weight rows the
//     whole tile is requested at once).
//   * Every load is a 1 KiB global_load_lds_dwordx4 (LDS DMA): a weight load
//     reads 1 KiB of one row (8 steps) or of two rows (4 steps each), an A
//     load 1 KiB of one A row.  Long row-contiguous runs keep the HBM pages
//     and channels busy, where 8 rows x 128 bytes per instruction does not;
//     the data goes straight to LDS, with no register round trip.
//   * The DMA writes lane i's 16 bytes to LDS slot i.  Lane i of a run of
//     row r reads the global chunk i ^ (r % 16), so LDS slot j of row r holds
//     chunk j ^ (r % 16): the MFMA operand reads (16 lanes = 16 rows, one
//     chunk each) then fall into 16 different bank groups.
//   * The stage order is rotated per tile, so concurrently running
//     workgroups read different K offsets of their rows.
//   * One workgroup barrier per stage publishes the stage and frees the
//     slot the next DMA refills.  The waves of a column block take the
//     stage's K steps round-robin; per step a wave dequantizes its 16x128
//     weight block exactly (v_cvt_scalef32_pk_bf16_fp8, scale 1.0), runs the
//     4 MFMA 16x16x32 BF16 per 16-row A block with the per-step K
//     relabelling of the other kernels (lane group g of MFMA q covers
//     physical k 32g+8q..+7), and folds the partial: acc = fma(s, p, acc).
//   * At the end the waves' partial tiles are added in LDS in wave order
//     (a fixed order: every run gives the same bits) and stored as BF16.
//   * Rows past n and m are read from clamped addresses and never stored;
//     steps past K in the last stage are read from a clamped address and
//     never used.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

using namespace dev;

template <int MB, int NBW, int SK, int NST, int WAVES, bool A8>
struct RingShape {
    static constexpr int NR = 16 * NBW;                 // weight rows
    static constexpr int AR = A8 ? 8 : 16 * MB;         // A rows staged
    static constexpr uint32_t W_ROW = SK * 128;         // bytes of a weight row per stage
    static constexpr uint32_t A_ROW = SK * 256;         // bytes of an A row per stage
    static constexpr uint32_t W_BYTES = NR * W_ROW;
    static constexpr uint32_t STAGE = W_BYTES + AR * A_ROW;
    static constexpr int NWI = W_BYTES / 1024;          // weight loads per stage
    static constexpr int NAI = AR * A_ROW / 1024;       // A loads per stage
    static constexpr int NI = (NWI + NAI) / WAVES;      // loads per wave per stage
    static constexpr int WK = WAVES / NBW;              // waves per column block
    static constexpr int SPW = (SK + WK - 1) / WK;      // max steps per wave per stage
    static constexpr bool valid = ring_shape_ok(MB, NBW, SK, NST, WAVES, A8);
};

// Issue this wave's NI loads of physical stage `ps` into ring slot `dst`.
// Lanes whose K step lies past K read their clamped stage-0 address.  Bit u
// of the wave-uniform `wmask` marks load u as a weight load: the weight is
// read once (the ring kernel's plans have one row tile), so it carries the
// non-temporal hint; A, read by every workgroup, does not.
template <int NI>
__device__ __forceinline__ void ring_issue(uint8_t *dst, uint32_t ps, uint32_t sk,
                                           uint32_t ksteps, const uint8_t *const *src,
                                           const uint32_t *stride, const uint32_t *lstep,
                                           const uint32_t *ldso, uint32_t wmask)
{
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const bool ok = ps * sk + lstep[u] < ksteps;
        const uint8_t *a = src[u] + (ok ? ps * stride[u] : 0u);
        if ((wmask >> u) & 1u)
            __builtin_amdgcn_global_load_lds(a, (lds_void_t *)(dst + ldso[u]), 16, 0, kNonTemporal);
        else
            __builtin_amdgcn_global_load_lds(a, (lds_void_t *)(dst + ldso[u]), 16, 0, 0);
    }
}

template <int MB, int NBW, int SK, int NST, int WAVES, bool A8>
__global__ __launch_bounds__(WAVES * 64) void w8a16_ring_kernel(GemmArgs g)
{
    using S = RingShape<MB, NBW, SK, NST, WAVES, A8>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float *const scl = reinterpret_cast<float *>(lds + NST * S::STAGE);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t tile = logical_wg(blockIdx.x, gridDim.x);
    const uint32_t m_tile = tile % g.m_tiles;
    const uint32_t n_tile = tile / g.m_tiles;
    const uint32_t n0 = n_tile * S::NR;
    const uint32_t m0 = m_tile * (16u * MB);
    const uint32_t ksteps = g.k / 128u;
    const uint32_t nst = (ksteps + SK - 1) / SK;
    const uint32_t rot = (tile * kRotStride) % nst;

    // The tile's scale row goes to LDS by DMA too, 64 steps per wave (the
    // planner keeps K/128 <= threads), ahead of the stage loads: waiting for
    // the first stage covers it.  (A plain load into registers here would
    // make the compiler drain every DMA in flight before its first use.)
    {
        const float *srow = g.scale + (size_t)(min(n0, g.n - 1u) / 128u) * ksteps;
        if (wave * 64u < ksteps) {
            const uint32_t t = min(wave * 64u + lane, ksteps - 1u);
            __builtin_amdgcn_global_load_lds(srow + t, (lds_void_t *)(scl + wave * 64u), 4, 0, 0);
        }
    }

    // ---- DMA sources of this wave's loads (load i = wave + WAVES * u) ----
    const uint8_t *src[S::NI];
    uint32_t stride[S::NI], lstep[S::NI], ldso[S::NI];
    uint32_t wmask = 0;
#pragma unroll
    for (int u = 0; u < S::NI; ++u) {
        const uint32_t i = wave + WAVES * u;
        if (i < (uint32_t)S::NWI) {
            wmask |= 1u << u;
            // 8 / SK weight rows per load, SK * 8 chunks (lanes) per row
            constexpr uint32_t LPR = SK * 8;
            const uint32_t r = i * (8 / SK) + lane / LPR;
            const uint32_t j = (lane % LPR) ^ (r & 15u);
            const uint32_t row = min(n0 + r, g.n - 1u);
            src[u] = g.w + (size_t)row * g.k + j * 16u;
            stride[u] = SK * 128u;
            lstep[u] = j / 8u;
            ldso[u] = i * 1024u;
        } else {
            // SK / 4 loads per A row, 64 chunks each
            const uint32_t ia = i - S::NWI;
            const uint32_t r = ia / (SK / 4), pp = ia % (SK / 4);
            const uint32_t j = (pp * 64u + lane) ^ (r & 15u);
            const uint32_t row = min(m0 + r, g.m - 1u);
            src[u] = g.a + (size_t)row * g.a_stride * 2u + j * 16u;
            stride[u] = SK * 256u;
            lstep[u] = j / 16u;
            ldso[u] = S::W_BYTES + r * S::A_ROW + pp * 1024u;
        }
    }

    // ---- MFMA operand reads: row rr = lane % 16, lane group gq = lane / 16
    // covers physical k 32gq..32gq+31 of a step (MFMA q takes 32gq+8q..+7).
    const uint32_t rr = lane & 15u, gq = lane >> 4;
    const uint32_t jb = wave / S::WK, kw = wave % S::WK;   // column block, step phase
    const uint32_t wrow = (16u * jb + rr) * S::W_ROW;
    uint32_t arow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const uint32_t r = A8 ? (rr & 7u) : 16u * b + rr;
        arow[b] = S::W_BYTES + r * S::A_ROW;
    }
    const uint32_t aswz = A8 ? (rr & 7u) : rr;   // (A row) % 16 of this lane's rows

    f32x4_t acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto phys = [&](uint32_t st) {
        const uint32_t x = st + rot;
        return x >= nst ? x - nst : x;
    };

    // Prologue: stages 0..NST-2, issued unconditionally (a stage past the
    // last reads clamped addresses into a slot nobody reads) so that the
    // number of loads in flight is fixed.  The waits below count only real
    // stages; an extra one can only make a wait longer.  (Filling the last
    // slot here as well measured slower: the LDS-DMA issue rate, not the
    // latency, bounds the start.)
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        ring_issue<S::NI>(lds + s * S::STAGE, phys(s), SK, ksteps, src, stride, lstep, ldso, wmask);

    uint32_t slot = 0;
    for (uint32_t st = 0; st < nst; ++st) {
        // Stages in flight behind st: min(nst - 1 - st, NST - 2).
        const uint32_t ahead = min(nst - 1u - st, (uint32_t)(NST - 2));
        if (ahead == 0)
            wait_vm<0>();
        else if (ahead == 1)
            wait_vm<S::NI>();
        else
            wait_vm<2 * S::NI>();
        barrier_lds();
        // Everyone is past stage st - 1: refill its slot.
        if (st + NST - 1 < nst) {
            const uint32_t fill = slot == 0 ? NST - 1 : slot - 1;
            ring_issue<S::NI>(lds + fill * S::STAGE, phys(st + NST - 1), SK, ksteps, src, stride,
                              lstep, ldso, wmask);
        }

        // The WK waves of column block jb take its logical steps
        // round-robin: wave kw takes steps kw, kw + WK, ...
        const uint8_t *stage = lds + slot * S::STAGE;
        const uint32_t ps = phys(st);
        const uint32_t s_first = (kw - st * SK) & (uint32_t)(S::WK - 1);
#pragma unroll
        for (int i = 0; i < S::SPW; ++i) {
            const uint32_t s = s_first + S::WK * i;
            const uint32_t t = ps * SK + s;
            if (s >= (uint32_t)SK || t >= ksteps)
                break;
            const u32x4_t r0 = *reinterpret_cast<const u32x4_t *>(
                stage + wrow + (((8u * s + 2u * gq) ^ rr) * 16u));
            const u32x4_t r1 = *reinterpret_cast<const u32x4_t *>(
                stage + wrow + (((8u * s + 2u * gq + 1u) ^ rr) * 16u));
            bf16x8_t af[MB][4];
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    af[b][q] = *reinterpret_cast<const bf16x8_t *>(
                        stage + arow[b] + (((16u * s + 4u * gq + q) ^ aswz) * 16u));
            bf16x8_t wb[4];
            dequant16(r0, wb[0], wb[1]);
            dequant16(r1, wb[2], wb[3]);
            const float sc = scl[t];
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                f32x4_t p = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[q], af[b][q], p, 0, 0, 0);
                acc[b].x = __builtin_fmaf(sc, p.x, acc[b].x);
                acc[b].y = __builtin_fmaf(sc, p.y, acc[b].y);
                acc[b].z = __builtin_fmaf(sc, p.z, acc[b].z);
                acc[b].w = __builtin_fmaf(sc, p.w, acc[b].w);
            }
        }
        slot = slot + 1 == NST ? 0 : slot + 1;
    }

    // ---- add the WK partials of each block in wave order, store C --------
    // Every wave has waited for all its loads (the last stage waits for 0),
    // so after this barrier no DMA writes into the ring any more.
    barrier_lds();
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);   // [WAVES][MB][64]
#pragma unroll
    for (int b = 0; b < MB; ++b)
        red[(wave * MB + b) * 64 + lane] = acc[b];
    barrier_lds();
    if constexpr (NBW * MB < WAVES) {
        // Fewer output tiles than waves: every thread adds one output's WK
        // partials (same wave order, same bits), so the tail is not left
        // to NBW * MB waves.
        constexpr uint32_t F = NBW * MB * 256u;
        const float *redf = reinterpret_cast<const float *>(lds);
        for (uint32_t f = threadIdx.x; f < F; f += WAVES * 64u) {
            // float f: component f % 4 of lane (f % 256) / 4 of pair f / 256
            const uint32_t pi = f / 256u, within = f % 256u, ln = within / 4u;
            const uint32_t j = pi / MB, b = pi % MB;
            float v[S::WK];
#pragma unroll
            for (int w = 0; w < S::WK; ++w)
                v[w] = redf[((j * S::WK + w) * MB + b) * 256u + within];
            float sum = v[0];
#pragma unroll
            for (int w = 1; w < S::WK; ++w)
                sum += v[w];
            const uint32_t row = m0 + 16u * b + (ln & 15u);
            const uint32_t col = n0 + 16u * j + 4u * (ln >> 4) + f % 4u;
            if (row < g.m && col < g.n)
                reinterpret_cast<uint16_t *>(g.c)[(size_t)row * g.c_stride + col] =
                    (uint16_t)f32_to_bf16_bits(sum);
        }
    } else {
        for (uint32_t pi = wave; pi < (uint32_t)(NBW * MB); pi += WAVES) {
            const uint32_t j = pi / MB, b = pi % MB;
            f32x4_t v[S::WK];
#pragma unroll
            for (int w = 0; w < S::WK; ++w)
                v[w] = red[((j * S::WK + w) * MB + b) * 64 + lane];
            f32x4_t sum = v[0];
#pragma unroll
            for (int w = 1; w < S::WK; ++w)
                sum += v[w];
            store_c4(g, sum, m0 + 16u * b + rr, n0 + 16u * j + 4u * gq);
        }
    }
}

template <int MB, int NBW, int SK, int NST, int WAVES, bool A8>
hipError_t launch_ring_t(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    if constexpr (!RingShape<MB, NBW, SK, NST, WAVES, A8>::valid) {
        (void)g, (void)p, (void)stream;
        return hipErrorInvalidValue;
    } else {
        auto kern = w8a16_ring_kernel<MB, NBW, SK, NST, WAVES, A8>;
        static std::atomic<uint64_t> lds_set{0};
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), p.lds_bytes,
                                 kMaxLdsBytes, lds_set);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, dim3(p.grid), dim3(p.block), p.lds_bytes, stream, g);
        return hipGetLastError();
    }
}

template <int MB, int NBW, int SK, int NST, bool A8>
hipError_t launch_ring_w(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.waves) {
    case 8: return launch_ring_t<MB, NBW, SK, NST, 8, A8>(g, p, stream);
    case 16: return launch_ring_t<MB, NBW, SK, NST, 16, A8>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int MB, int NBW, int SK, bool A8>
hipError_t launch_ring_n(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.depth) {
    case 2: return launch_ring_w<MB, NBW, SK, 2, A8>(g, p, stream);
    case 3: return launch_ring_w<MB, NBW, SK, 3, A8>(g, p, stream);
    case 4: return launch_ring_w<MB, NBW, SK, 4, A8>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int MB, int NBW, bool A8>
hipError_t launch_ring_s(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    switch (p.stage_steps) {
    case 4: return launch_ring_n<MB, NBW, 4, A8>(g, p, stream);
    case 8: return launch_ring_n<MB, NBW, 8, A8>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_ring(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    const bool a8 = (p.flags & W8A16_FLAG_A8) != 0;
    switch (p.m_blocks * 100 + p.n_blocks * 10 + (a8 ? 1 : 0)) {
    case 111: return launch_ring_s<1, 1, true>(g, p, stream);
    case 121: return launch_ring_s<1, 2, true>(g, p, stream);
    case 141: return launch_ring_s<1, 4, true>(g, p, stream);
    case 110: return launch_ring_s<1, 1, false>(g, p, stream);
    case 120: return launch_ring_s<1, 2, false>(g, p, stream);
    case 140: return launch_ring_s<1, 4, false>(g, p, stream);
    case 210: return launch_ring_s<2, 1, false>(g, p, stream);
    case 220: return launch_ring_s<2, 2, false>(g, p, stream);
    case 240: return launch_ring_s<2, 4, false>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace w8a16
