// Internal declarations shared by the planner and the launch code.
#pragma once

#include <stdint.h>

#include "w8a16.h"

namespace w8a16 {

constexpr uint32_t kKStep = 128;        // K width of one FP8 scale block
constexpr uint32_t kWaves = 4;          // waves per stream-kernel workgroup
constexpr uint32_t kWBlockBytes = 16 * 128;      // 16 weight rows x one K step (FP8)
constexpr uint32_t kABlockBytes = 16 * 128 * 2;  // 16 A rows x one K step (BF16)
constexpr uint32_t kAccBytes = 64 * 4 * 4;       // one 16x16 FP32 MFMA tile
constexpr uint32_t kDefaultCUs = 256;            // MI355X
// Dynamic LDS a plan may use: the 160 KiB of a gfx950 CU less room for the
// kernels' small static __shared__ variables.
constexpr uint32_t kMaxLdsBytes = 160 * 1024 - 256;
constexpr uint32_t kTileMaxSteps = 64;
// Split-K arrival counters sit 256 bytes apart (one per tile), so that no
// two tiles' atomics meet in one cache line.
constexpr uint32_t kCounterStride = 64;           // tile kernel: K steps per split (one per lane)

// LDS of the tile kernel for a (16 * m_blocks) x (16 * n_blocks) C tile:
// a_stages buffers of one K step of A (16 * m_blocks rows x 256 bytes of
// BF16), w_stages buffers of one K step of the FP8 weight (16 * n_blocks
// rows x 128 bytes) and the split's scale row (at most 64 floats).
constexpr uint32_t tile_lds_bytes(uint32_t m_blocks, uint32_t n_blocks, uint32_t w_stages,
                                  uint32_t a_stages)
{
    return a_stages * 16 * m_blocks * 256 + w_stages * 16 * n_blocks * 128 + 256;
}

// LDS of the wide tile kernel (128 x 256 C tile, m_blocks 8, n_blocks 16):
// three K steps of weight (256 rows x 128 bytes), three K halves of A (128
// rows x 128 bytes) and the two 128-column blocks' scale rows (64 floats
// each).
constexpr uint32_t wide_lds_bytes() { return 3 * 256 * 128 + 3 * 128 * 128 + 2 * 256; }
constexpr uint32_t kWideMBlocks = 8, kWideNBlocks = 16;

// Built tile-kernel ring sizes (weight buffers = depth, A buffers =
// a_depth) per tile shape; tiles are 64 or 128 rows by 64 or 128 columns.
// The list is the dispatch table of the tile kernel's launcher.
#define W8A16_TILE_VARIANTS(X)                                                        \
    X(8, 4, 4, 2) X(8, 4, 6, 2) X(8, 4, 8, 2) X(8, 4, 4, 3) X(8, 4, 6, 3)             \
    X(8, 8, 3, 2) X(8, 8, 4, 2) X(8, 8, 5, 2) X(8, 8, 3, 3)                           \
    X(4, 4, 6, 2) X(4, 4, 8, 2) X(4, 4, 6, 3) X(4, 4, 8, 3) X(4, 4, 8, 4)             \
    X(4, 4, 6, 5) X(4, 4, 4, 6) X(4, 4, 6, 6)                                         \
    X(4, 8, 4, 2) X(4, 8, 6, 2) X(4, 8, 4, 3) X(4, 8, 6, 3) X(4, 8, 4, 4)             \
    X(4, 8, 5, 4) X(4, 8, 4, 5) X(4, 8, 3, 5) X(4, 8, 3, 6)

constexpr uint32_t tile_variant_key(uint32_t m_blocks, uint32_t n_blocks, uint32_t depth,
                                    uint32_t a_depth)
{
    return ((m_blocks * 16 + n_blocks) * 16 + depth) * 16 + a_depth;
}

constexpr bool tile_depth_built(uint32_t m_blocks, uint32_t n_blocks, uint32_t depth,
                                uint32_t a_depth)
{
#define W8A16_TILE_KEY_MATCH(MB, NB, D, AD) || key == tile_variant_key(MB, NB, D, AD)
    const uint32_t key = tile_variant_key(m_blocks, n_blocks, depth, a_depth);
    return false W8A16_TILE_VARIANTS(W8A16_TILE_KEY_MATCH);
#undef W8A16_TILE_KEY_MATCH
}

// Tile kernel wave counts: 4 (one wave per SIMD), 8 (two groups splitting
// every K step), and 6 or 10 (those plus two producer waves that only issue
// the LDS DMA).  Variants that would spill registers are not built: with
// producers, a SIMD holds three waves of the 8-wave layout (10 waves), which
// fits the 128-row tile only at 64 columns, and the 6-wave 128 x 128 tile
// fits only two A buffers.  A producer wave waits on up to depth - 2 steps
// of its ring (n_blocks * 2 loads each), which the 6-bit vmcnt must hold.
constexpr bool tile_variant_ok(uint32_t m_blocks, uint32_t n_blocks, uint32_t depth,
                               uint32_t a_stages, uint32_t waves)
{
    if (waves == 4 || waves == 8)
        return true;
    if (n_blocks * 2 * (depth - 2) > 63 || m_blocks * 4 * (a_stages - 2) > 63)
        return false;
    if (m_blocks == 4)
        return waves == 6 || waves == 10;
    if (waves == 6)
        return n_blocks == 4 || a_stages == 2;
    if (waves == 10)
        return n_blocks == 4;
    return false;
}

// Ring kernel geometry, shared by the planner and the kernel dispatch.  A
// workgroup owns nbw 16-column blocks and mb 16-row blocks of C (a8: m <= 8,
// only 8 A rows staged) over all of K, in stages of sk K steps; a ring of
// nst stages is in flight.  One stage holds 16 * nbw weight rows x sk * 128
// bytes and the A rows x sk * 256 bytes.
constexpr uint32_t ring_a_rows(uint32_t mb, bool a8) { return a8 ? 8 : 16 * mb; }

constexpr uint32_t ring_stage_bytes(uint32_t mb, uint32_t nbw, uint32_t sk, bool a8)
{
    return sk * (16 * nbw * 128 + ring_a_rows(mb, a8) * 256);
}

// LDS of the ring kernel: the ring plus the tile's scale row (K/128 floats,
// loaded 64 at a time).
constexpr uint32_t ring_lds_bytes(uint32_t mb, uint32_t nbw, uint32_t sk, uint32_t nst, bool a8,
                                  uint32_t ksteps)
{
    return nst * ring_stage_bytes(mb, nbw, sk, a8) + (ksteps + 63) / 64 * 256;
}

// Shapes the ring kernel is built for: every stage splits evenly into 1 KiB
// DMA loads over the waves, the waves split evenly over the column blocks,
// the ring fits in LDS (with room for a small scale row) and can hold the
// waves' partial tiles at the end.
constexpr bool ring_shape_ok(uint32_t mb, uint32_t nbw, uint32_t sk, uint32_t nst, uint32_t waves,
                             bool a8)
{
    const bool mb_ok = mb == 1 || mb == 2;
    const bool nb_ok = nbw == 1 || nbw == 2 || nbw == 4;
    const bool sk_ok = sk == 4 || sk == 8;
    const bool nst_ok = nst >= 2 && nst <= 4;
    const bool w_ok = waves == 8 || waves == 16;
    if (!(mb_ok && nb_ok && sk_ok && nst_ok && w_ok) || (a8 && mb != 1))
        return false;
    const uint32_t loads = (16 * nbw * sk * 128 + ring_a_rows(mb, a8) * sk * 256) / 1024;
    const uint32_t ring = nst * ring_stage_bytes(mb, nbw, sk, a8);
    return waves % nbw == 0 && loads % waves == 0 && ring + 1024 <= kMaxLdsBytes &&
           waves * mb * 1024 <= ring;
}

// W4A4 MX GEMV: most rows and largest K.  LDS of the persistent kernel: A
// (16 m_blocks rows padded by 16 bytes), its scale bytes (rounded up to
// 256) and two partial 16 x 16 tiles per wave and row block.
constexpr uint32_t kW4a4MaxM = 64;
constexpr uint32_t kW4a4MaxK = 1u << 24;          // K and A pitch, in FP4 elements
constexpr uint32_t w4a4_ps_a_bytes(uint32_t m_blocks, uint32_t k)
{
    return m_blocks * 16 * (k / 2 + 16);
}
constexpr uint32_t w4a4_ps_s_bytes(uint32_t m_blocks, uint32_t k)
{
    return (m_blocks * 16 * (k / 32) + 255) / 256 * 256;
}
constexpr uint32_t w4a4_ps_lds_bytes(uint32_t m_blocks, uint32_t k, uint32_t waves)
{
    return w4a4_ps_a_bytes(m_blocks, k) + w4a4_ps_s_bytes(m_blocks, k) + waves * 2 * m_blocks * 1024;
}
// The persistent kernel is planned for weights of at least this many 16-row
// tiles per CU.
constexpr uint32_t kW4a4PsMinTilesPerCu = 2;
// Tiled W4A4 variants that are built: a wave holds two groups of 4 K steps
// of its mb + nb operand blocks in registers, which fits the 128 VGPRs of a
// 16-wave workgroup for one block each and the 256 of an 8-wave workgroup
// for up to four blocks; 4 waves take any shape.
constexpr bool w4a4_variant_ok(uint32_t mb, uint32_t nb, uint32_t waves)
{
    return waves == 4 || (waves == 8 && mb + nb <= 4) || (waves == 16 && mb + nb <= 2);
}

int check_args(uint32_t m, uint32_t n, uint32_t k, uint32_t a_row_stride,
               uint32_t c_row_stride);
int check_args_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t a_row_stride,
                    uint32_t c_row_stride);
int make_plan_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out);
int make_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out);
int plan_finalize(uint32_t m, uint32_t n, uint32_t k, w8a16_plan_t *p);
int make_plan_w8a8(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out);
int plan_batched(const w8a16_gemm_desc_t *descs, uint32_t count, uint32_t cu_count,
                 w8a16_plan_t *out);
// Replace the "w8a16_gemm" prefix of the last error by `name`.
int fail_with_name(int status, const char *name);
// Prefix the last error with "w8a16_gemm_batched: descriptor <index>: ".
int fail_at(int status, uint32_t index);
const char *status_string(int status);
// Why the calling thread's last successful default plan was chosen (the
// planner rule that picked kernel and tile), for the plan log.
const char *plan_reason();
const char *last_error();
void set_last_error(const char *msg);
int fail(int status, const char *msg);

}  // namespace w8a16
