// Argument checks, launch planning and status text for the W8A16 GEMM.
//
// Pure host code with no HIP dependency, so the checks and the plans can be
// graded on a machine without a GPU.
//
// The argument rules are those of `w8a16_gemm_pipelined_m32_strided` on the
// page "w8a16_gemm_pipelined_m32.rs" (its `ensure!` checks, in their order):
// m >= 1; k a positive multiple of 128 (one FP8 scale block per K step);
// both pitches covering the used extents; a_row_stride a multiple of 8 so
// A rows stay 16-byte aligned.  n == 0 and null pointers are rejected after
// those, which the page does not check.
//
// The tile rule keeps the page's idea (small m streams the weight once,
// large m uses a big row tile; `w8a16_pipelined_prefers_m32`,
// `w8a16_pipelined_prefers_m64`, `w8a16_gemm_pipelined_by_m`), re-derived
// for MI355X: 256 CUs, 64-wide waves, 16x16x32 BF16 MFMA.

#include "plan.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

namespace w8a16 {

namespace {
thread_local std::string g_last_error;
thread_local char g_plan_reason[256];

void set_reason(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void set_reason(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_plan_reason, sizeof g_plan_reason, fmt, ap);
    va_end(ap);
}
}  // namespace

const char *plan_reason() { return g_plan_reason; }

void set_last_error(const char *fmt_msg) { g_last_error = fmt_msg ? fmt_msg : ""; }

const char *last_error() { return g_last_error.c_str(); }

int fail(int status, const char *msg)
{
    set_last_error(msg);
    return status;
}

int check_args(uint32_t m, uint32_t n, uint32_t k, uint32_t a_row_stride,
               uint32_t c_row_stride)
{
    char buf[256];
    if (m < 1)
        return fail(W8A16_ERR_M_ZERO, "w8a16_gemm: m=0 has no rows to compute");
    if (k < kKStep || k % kKStep != 0) {
        snprintf(buf, sizeof buf,
                 "w8a16_gemm: K=%u must be a positive multiple of %u (one FP8 "
                 "scale block per K-step)", k, kKStep);
        return fail(W8A16_ERR_K_NOT_MULT_128, buf);
    }
    if (a_row_stride < k || c_row_stride < n) {
        snprintf(buf, sizeof buf,
                 "w8a16_gemm: row pitches (a=%u, c=%u) must cover the used "
                 "extents (k=%u, n=%u)", a_row_stride, c_row_stride, k, n);
        return fail(W8A16_ERR_PITCH_TOO_SHORT, buf);
    }
    if (a_row_stride % 8 != 0) {
        snprintf(buf, sizeof buf,
                 "w8a16_gemm: a_row_stride=%u must keep rows 16B-aligned "
                 "(multiple of 8 elements)", a_row_stride);
        return fail(W8A16_ERR_A_STRIDE_ALIGN, buf);
    }
    if (n < 1)
        return fail(W8A16_ERR_N_ZERO, "w8a16_gemm: n=0 has no columns to compute");
    return W8A16_OK;
}

static uint32_t div_up(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

static bool stream_shape_supported(uint32_t mb, uint32_t nb)
{
    switch (mb * 100 + nb) {
    case 101: case 102: case 103: case 104: case 108:
    case 201: case 202: case 204: case 208:
    case 401: case 402:
        return true;
    default:
        return false;
    }
}

// Bytes (per 128 of K) a CU requests for a stream tile of mb 16-row and
// nb 16-column blocks: the tile's A rows (BF16) and weight rows (FP8),
// times the rounds of tiles each CU runs.
static uint64_t stream_tile_cost(uint32_t m, uint32_t nb16, uint32_t cus, uint32_t mb,
                                 uint32_t nb)
{
    const uint64_t t = (uint64_t)div_up(m, 16 * mb) * div_up(nb16, nb);
    return (t + cus - 1) / cus * (32ull * mb + 16ull * nb);
}

struct StreamTile {
    uint32_t mb, nb;
    uint64_t cost;
};

// The stream tile with the lowest stream_tile_cost; ties go to more rows,
// then more columns.  32 x 128 tiles are left out: they run only as four
// waves, measured 1.9x slower than 32 x 64 tiles at the same rows.
static StreamTile cheapest_stream_tile(uint32_t m, uint32_t nb16, uint32_t cus)
{
    StreamTile best = {0, 0, ~0ull};
    const uint32_t mbs[3] = {4, 2, 1}, nbs[5] = {8, 4, 3, 2, 1};
    for (uint32_t mb : mbs)
        for (uint32_t nb : nbs) {
            if (!stream_shape_supported(mb, nb) || (mb == 2 && nb == 8))
                continue;
            const uint64_t c = stream_tile_cost(m, nb16, cus, mb, nb);
            if (c < best.cost)
                best = {mb, nb, c};
        }
    return best;
}

static bool w8a8_shape_supported(uint32_t mb, uint32_t nb)
{
    switch (mb * 100 + nb) {
    case 101: case 102: case 103: case 104:
    case 201: case 202: case 204:
    case 401: case 402:
        return true;
    default:
        return false;
    }
}

// W8A8 kernel LDS: per wave one K step of its weight and A blocks (16 rows x
// 128 bytes each), reused for the wave-order reduction of the partial tiles.
static uint32_t w8a8_lds_bytes(uint32_t mb, uint32_t nb, uint32_t waves)
{
    const uint32_t staging = waves * (nb + mb) * 2048u;
    const uint32_t reduce = waves * nb * mb * kAccBytes;
    return staging > reduce ? staging : reduce;
}

static bool w4a4_shape_supported(uint32_t mb, uint32_t nb)
{
    return (mb == 1 || mb == 2 || mb == 4) && (nb == 1 || nb == 2 || nb == 4) &&
           !(mb == 4 && nb == 4);
}

static bool tile_shape_supported(uint32_t mb, uint32_t nb)
{
    return ((mb == 4 || mb == 8) && (nb == 4 || nb == 8)) ||
           (mb == kWideMBlocks && nb == kWideNBlocks);
}

int plan_finalize(uint32_t m, uint32_t n, uint32_t k, w8a16_plan_t *p)
{
    char buf[256];
    if (!p)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_plan: null plan");
    int st = check_args(m, n, k, k, n);
    if (st != W8A16_OK)
        return st;
    const uint32_t ksteps = k / kKStep;
    if (p->cu_count == 0)
        p->cu_count = kDefaultCUs;
    if (p->kernel == W8A16_KERNEL_STREAM) {
        if (!stream_shape_supported(p->m_blocks, p->n_blocks)) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: stream kernel has no (m_blocks=%u, n_blocks=%u) "
                     "variant", p->m_blocks, p->n_blocks);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        if (p->depth != 1 && p->depth != 2 && p->depth != 4) {
            snprintf(buf, sizeof buf, "w8a16_plan: depth=%u must be 1, 2 or 4", p->depth);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        if (p->flags & ~(uint32_t)(W8A16_FLAG_DIRECT | W8A16_FLAG_XCD_LOCAL)) {
            snprintf(buf, sizeof buf, "w8a16_plan: unknown flags 0x%x", p->flags);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        if (p->waves != 4 && p->waves != 8 && p->waves != 16) {
            snprintf(buf, sizeof buf, "w8a16_plan: waves=%u must be 4, 8 or 16", p->waves);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        p->block = p->waves * 64;
        p->stage_steps = 0;
        p->a_depth = 0;
        const bool direct = (p->flags & W8A16_FLAG_DIRECT) != 0;
        uint32_t per_wave = p->n_blocks * kWBlockBytes + (direct ? 0u : p->m_blocks * kABlockBytes);
        uint32_t staging = p->waves * per_wave;
        uint32_t reduce = p->waves * p->n_blocks * p->m_blocks * kAccBytes;
        p->lds_bytes = staging > reduce ? staging : reduce;
        if (p->lds_bytes > kMaxLdsBytes) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: %u bytes of LDS per workgroup exceed the %u available",
                     p->lds_bytes, kMaxLdsBytes);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
    } else if (p->kernel == W8A16_KERNEL_RING) {
        // m <= 8 stages 8 A rows; the flag is derived, not chosen
        const bool a8 = m <= 8 && p->m_blocks == 1;
        p->flags = a8 ? (uint32_t)W8A16_FLAG_A8 : 0u;
        if (!ring_shape_ok(p->m_blocks, p->n_blocks, p->stage_steps, p->depth, p->waves, a8)) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: ring kernel has no (m_blocks=%u, n_blocks=%u, stage_steps=%u, "
                     "depth=%u, waves=%u) variant", p->m_blocks, p->n_blocks, p->stage_steps,
                     p->depth, p->waves);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        if (ksteps > p->waves * 64u || p->splits != 1) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: ring kernel needs K/128=%u at most %u and splits=1 (got %u)",
                     ksteps, p->waves * 64u, p->splits);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        p->block = p->waves * 64;
        p->a_depth = 0;
        p->lds_bytes = ring_lds_bytes(p->m_blocks, p->n_blocks, p->stage_steps, p->depth, a8, ksteps);
        if (p->lds_bytes > kMaxLdsBytes) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: %u bytes of LDS per workgroup exceed the %u available",
                     p->lds_bytes, kMaxLdsBytes);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
    } else if (p->kernel == W8A16_KERNEL_TILE) {
        if (!tile_shape_supported(p->m_blocks, p->n_blocks)) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: tile kernel has no (m_blocks=%u, n_blocks=%u) "
                     "variant", p->m_blocks, p->n_blocks);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        if (p->m_blocks == kWideMBlocks && p->n_blocks == kWideNBlocks) {
            // the wide tile: fixed rings (3 weight steps, 3 A halves), 4 waves
            if (p->depth == 0)
                p->depth = 3;
            if (p->a_depth == 0)
                p->a_depth = 3;
            if (p->waves == 0)
                p->waves = 4;
            if (p->flags != 0 || p->depth != 3 || p->a_depth != 3 || p->waves != 4) {
                snprintf(buf, sizeof buf,
                         "w8a16_plan: the 128 x 256 tile takes depth 3, a_depth 3, 4 waves and "
                         "no flags (depth=%u, a_depth=%u, waves=%u, flags=0x%x)", p->depth,
                         p->a_depth, p->waves, p->flags);
                return fail(W8A16_ERR_BAD_PLAN, buf);
            }
            p->stage_steps = 0;
            p->block = 256;
            p->lds_bytes = wide_lds_bytes();
        } else {
            if (p->flags != 0 ||
                (p->waves != 0 && p->waves != 4 && p->waves != 6 && p->waves != 8 &&
                 p->waves != 10)) {
                snprintf(buf, sizeof buf,
                         "w8a16_plan: tile kernel takes no flags and 4, 6, 8 or 10 waves "
                         "(flags=0x%x, waves=%u)", p->flags, p->waves);
                return fail(W8A16_ERR_BAD_PLAN, buf);
            }
            // Built (weight buffers, A buffers) pairs; all fit in LDS.
            if (p->a_depth == 0)
                p->a_depth = 2;
            const uint32_t ast = p->a_depth;
            if (!tile_depth_built(p->m_blocks, p->n_blocks, p->depth, ast)) {
                snprintf(buf, sizeof buf,
                         "w8a16_plan: tile kernel has no depth=%u variant for m_blocks=%u, "
                         "n_blocks=%u with %u A buffers", p->depth, p->m_blocks, p->n_blocks,
                         ast);
                return fail(W8A16_ERR_BAD_PLAN, buf);
            }
            if (p->waves == 0)
                p->waves = 4;
            if (!tile_variant_ok(p->m_blocks, p->n_blocks, p->depth, ast, p->waves)) {
                snprintf(buf, sizeof buf,
                         "w8a16_plan: tile kernel has no %u-wave variant for m_blocks=%u, "
                         "n_blocks=%u with %u A buffers", p->waves, p->m_blocks, p->n_blocks,
                         ast);
                return fail(W8A16_ERR_BAD_PLAN, buf);
            }
            p->stage_steps = 0;
            p->block = p->waves * 64;
            p->lds_bytes = tile_lds_bytes(p->m_blocks, p->n_blocks, p->depth, ast);
        }
        if (p->lds_bytes > kMaxLdsBytes) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: %u bytes of LDS per workgroup exceed the %u available",
                     p->lds_bytes, kMaxLdsBytes);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
    } else if (p->kernel == W8A16_KERNEL_W8A8) {
        if (!w8a8_shape_supported(p->m_blocks, p->n_blocks) ||
            (p->waves != 4 && p->waves != 8 && p->waves != 16) ||
            (p->waves == 16 && p->m_blocks * p->n_blocks > 2) || p->flags != 0 ||
            p->splits != 1) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: W8A8 kernel has no (m_blocks=%u, n_blocks=%u, waves=%u, "
                     "flags=0x%x, splits=%u) variant", p->m_blocks, p->n_blocks, p->waves,
                     p->flags, p->splits);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        p->depth = 2;
        p->stage_steps = 0;
        p->a_depth = 0;
        p->block = p->waves * 64;
        p->lds_bytes = w8a8_lds_bytes(p->m_blocks, p->n_blocks, p->waves);
        if (p->lds_bytes > kMaxLdsBytes) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: %u bytes of LDS per workgroup exceed the %u available",
                     p->lds_bytes, kMaxLdsBytes);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
    } else if (p->kernel == W8A16_KERNEL_W4A4) {
        if (!w4a4_shape_supported(p->m_blocks, p->n_blocks) ||
            !w4a4_variant_ok(p->m_blocks, p->n_blocks, p->waves) || p->flags != 0 ||
            p->splits != 1 || m > kW4a4MaxM) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: W4A4 kernel has no (m_blocks=%u, n_blocks=%u, waves=%u, "
                     "flags=0x%x, splits=%u) variant for m=%u (at most %u rows)", p->m_blocks,
                     p->n_blocks, p->waves, p->flags, p->splits, m, kW4a4MaxM);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        p->depth = 2;
        p->stage_steps = 0;
        p->a_depth = 0;
        p->block = p->waves * 64;
        p->lds_bytes = p->waves * p->m_blocks * p->n_blocks * kAccBytes;
    } else if (p->kernel == W8A16_KERNEL_W4A4_PS) {
        if ((p->m_blocks != 1 && p->m_blocks != 2 && p->m_blocks != 4) || 16 * p->m_blocks < m ||
            (p->waves != 4 && p->waves != 8 && p->waves != 16) || p->flags != 0 ||
            p->splits != 1 || m > kW4a4MaxM) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: persistent W4A4 kernel needs m_blocks 1, 2 or 4 covering "
                     "m=%u (at most %u rows), 4, 8 or 16 waves, no flags and no split "
                     "(m_blocks=%u, waves=%u, flags=0x%x, splits=%u)", m, kW4a4MaxM,
                     p->m_blocks, p->waves, p->flags, p->splits);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        p->n_blocks = 1;
        p->depth = 3;
        p->stage_steps = 0;
        p->a_depth = 0;
        p->block = p->waves * 64;
        p->lds_bytes = w4a4_ps_lds_bytes(p->m_blocks, k, p->waves);
        if (p->lds_bytes > kMaxLdsBytes) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: the persistent W4A4 kernel's %u bytes of staged activations "
                     "and partial tiles exceed the %u bytes of LDS", p->lds_bytes, kMaxLdsBytes);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
    } else {
        snprintf(buf, sizeof buf, "w8a16_plan: unknown kernel %u", p->kernel);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    if (p->splits < 1 || p->splits > ksteps) {
        snprintf(buf, sizeof buf,
                 "w8a16_plan: splits=%u must be in 1..%u (K steps)", p->splits, ksteps);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    // Equal step counts per split; the count of splits actually needed may
    // shrink (e.g. 32 steps in 5 splits of 7 -> 5 splits, the last with 4).
    p->steps_per_split = div_up(ksteps, p->splits);
    p->splits = div_up(ksteps, p->steps_per_split);
    if (p->kernel == W8A16_KERNEL_TILE && p->steps_per_split > kTileMaxSteps) {
        snprintf(buf, sizeof buf,
                 "w8a16_plan: tile kernel splits of %u K steps exceed %u; use splits >= %u",
                 p->steps_per_split, kTileMaxSteps, div_up(ksteps, kTileMaxSteps));
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    p->m_tiles = div_up(m, 16 * p->m_blocks);
    p->n_tiles = div_up(n, 16 * p->n_blocks);
    uint64_t tiles = (uint64_t)p->m_tiles * p->n_tiles;
    uint64_t grid = tiles * p->splits;
    if (grid > 0x7fffffffull) {
        snprintf(buf, sizeof buf, "w8a16_plan: grid of %llu workgroups is too large",
                 (unsigned long long)grid);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    p->grid = (uint32_t)grid;
    if (p->kernel == W8A16_KERNEL_W4A4_PS) {
        // one workgroup per CU, each with an equal share of the 16-row
        // weight tiles (fewer workgroups than CUs for fewer tiles)
        const uint32_t tiles16 = div_up(n, 16);
        p->grid = p->cu_count < tiles16 ? p->cu_count : tiles16;
        p->workspace_bytes = 0;
        p->counter_count = 0;
        return W8A16_OK;
    }
    if (p->flags & W8A16_FLAG_XCD_LOCAL) {
        // The splits of a tile are consecutive logical workgroups, and each
        // XCD runs a contiguous range of grid / 8 of them: the ranges must
        // hold whole tiles.
        if (p->kernel != W8A16_KERNEL_STREAM || p->splits < 2 || p->grid % 8 != 0 ||
            (p->grid / 8) % p->splits != 0) {
            snprintf(buf, sizeof buf,
                     "w8a16_plan: XCD-local split publication needs the stream kernel, "
                     "splits >= 2 and a grid of 8 equal ranges of whole tiles (splits=%u, "
                     "grid=%u)", p->splits, p->grid);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
    }
    if (p->splits > 1 && p->kernel == W8A16_KERNEL_TILE) {
        // whole FP32 tiles per split, added by a second kernel
        p->workspace_bytes = (uint64_t)p->splits * p->m_tiles * 16 * p->m_blocks *
                             p->n_tiles * 16 * p->n_blocks * 4;
        p->counter_count = 0;
    } else if (p->splits > 1) {
        p->workspace_bytes = grid * (uint64_t)p->m_blocks * p->n_blocks * kAccBytes;
        p->counter_count = (uint32_t)tiles * kCounterStride;
    } else {
        p->workspace_bytes = 0;
        p->counter_count = 0;
    }
    return W8A16_OK;
}

int make_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out)
{
    if (!out)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_plan: null plan");
    int st = check_args(m, n, k, k, n);
    if (st != W8A16_OK)
        return st;
    w8a16_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.cu_count = cu_count ? cu_count : kDefaultCUs;
    const uint32_t ksteps = k / kKStep;
    const uint32_t nb16 = div_up(n, 16);

    // Above 32 rows a weight larger than 16 MiB goes through the tile
    // kernel (one L2 pass of the weight per 64-row tile; measured on
    // MI355X: 48 x 8192 x 8192 22 vs 32 us streaming).  Smaller weights
    // stream up to 64 rows, and up to 128 rows while the stream tile that
    // asks each CU for the fewest bytes needs one round of tiles
    // (65 x 4096 x 4096 12.8 vs 15.6 us in the tile kernel, 128 x 4096 x
    // 4096 14.9 vs 16.8, 96 x 2048 x 4096 9.9 vs 12.2; two rounds lose:
    // 128 x 6144 x 2048 15.5 vs 12.2).
    const uint64_t wbytes = (uint64_t)n * k;
    StreamTile st16 = {1, 1, 0};
    if (m > 16)
        st16 = cheapest_stream_tile(m, nb16, p.cu_count);
    const char *why = "";
    const bool stream_fits = m <= 128 && wbytes <= (16ull << 20) &&
                             (uint64_t)div_up(m, 16 * st16.mb) * div_up(nb16, st16.nb) <= p.cu_count;
    if (m > 128 || (m > 32 && wbytes > (16ull << 20)) || (m > 64 && !stream_fits)) {
        // 64-row tiles up to 128 rows, 128-row tiles above (fewer weight
        // passes).  The grid is one workgroup per CU: K is split until the
        // tiles fill the CUs, with 128-column tiles when that leaves each
        // split 16 or more K steps, else 64-column tiles (measured best at
        // 48..128 rows over 4096- and 8192-square weights).  Ring sizes
        // and waves are the measured best per tile shape.
        p.kernel = W8A16_KERNEL_TILE;
        p.flags = 0;
        p.m_blocks = m <= 128 ? 4 : 8;
        why = m > 128 ? "m > 128: tile kernel, 128-row tiles"
              : (m > 32 && wbytes > (16ull << 20))
                  ? "m > 32 over a weight above 16 MiB: tile kernel, 64-row tiles"
                  : "m > 64 and no stream tile fits one round per CU: tile kernel";
        const uint32_t m_tiles = div_up(m, 16 * p.m_blocks);
        auto splits_fill = [&](uint32_t tiles) {
            uint32_t sp = 1;
            while (tiles * sp * 2 <= p.cu_count && sp * 2 <= ksteps)
                sp *= 2;
            return sp;
        };
        p.n_blocks = 8;
        p.splits = splits_fill(m_tiles * div_up(n, 128));
        if (ksteps / p.splits < 16) {
            p.n_blocks = 4;
            p.splits = splits_fill(m_tiles * div_up(n, 64));
        }
        if (p.m_blocks == 4) {
            p.depth = 4;
            p.a_depth = p.n_blocks == 8 ? 4 : 6;
            p.waves = p.n_blocks == 8 ? 10 : 8;
        } else {
            p.depth = p.n_blocks == 8 ? 3 : 4;
            p.a_depth = 2;
            p.waves = 8;
        }
        if (p.splits < div_up(ksteps, kTileMaxSteps))
            p.splits = div_up(ksteps, kTileMaxSteps);
        // 65..128 rows: one 128 x 128 tile per column block, so the weight
        // crosses HBM once, when the K splits that fill the CUs keep 16 or
        // more K steps each (measured on MI355X, us per call, two 64-row
        // tiles -> one 128-row tile with 4 splits: 128 x 8192 x 8192
        // 32.1-32.9 -> 31.1-31.3, 96 x 8192 x 8192 31.3-31.6 -> 30.6-30.8,
        // 72 x 8192 x 8192 30.5-30.7 -> 29.4-30.1; with 8 steps per split
        // it is even at 128 x 8192 x 4096 and loses at 128 x 4096 x 8192,
        // 21.5-22.0 -> 25.2-26.2).
        if (m > 64 && m <= 128) {
            const uint32_t sp = splits_fill(div_up(n, 128));
            if (ksteps / sp >= 16 && sp >= div_up(ksteps, kTileMaxSteps)) {
                p.m_blocks = 8;
                p.n_blocks = 8;
                p.splits = sp;
                p.depth = 3;
                p.a_depth = 3;
                p.waves = 8;
                why = "65..128 rows with K splits of 16 or more steps: tile kernel, one 128-row "
                      "tile (the weight read once)";
            }
        }
    } else {
        // Small m: the weight-streaming kernel.  Measured on MI355X, the
        // best plans give each CU about one workgroup tile, enough waves
        // that every wave has only a few K steps (so a CU's whole share of
        // the weight is requested in about one memory round trip), and no K
        // split while the tiles fill the CUs: the last split's tail (its
        // partial reads) costs more than the A bytes a split saves.  Narrow
        // N splits K (below).
        p.kernel = W8A16_KERNEL_STREAM;
        p.depth = 1;
        p.flags = 0;
        p.m_blocks = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
        why = "small m: stream kernel, widest column tile giving 3/4 of the CUs a tile";
        uint32_t m_tiles = div_up(m, 16 * p.m_blocks);
        const uint32_t fill = (3 * p.cu_count) / 4;
        uint32_t nbw = 1;
        const uint32_t cands[3] = {4, 2, 1};
        for (uint32_t c : cands) {
            if (!stream_shape_supported(p.m_blocks, c))
                continue;
            if (div_up(nb16, c) * m_tiles >= fill) {
                nbw = c;
                break;
            }
        }
        // 48-column tiles when they fill the CUs' last round of tiles
        // clearly better than the choice above (12288 columns: 256 tiles of
        // 48 instead of 192 of 64; measured 14.9 vs 15.4 us at 16 x 12288 x
        // 5120).
        auto occupancy = [&](uint32_t c) {
            const uint64_t t = (uint64_t)div_up(nb16, c) * m_tiles;
            const uint64_t rounds = (t + p.cu_count - 1) / p.cu_count;
            return (double)t / (double)(rounds * p.cu_count);
        };
        if (stream_shape_supported(p.m_blocks, 3) && nbw > 1 &&
            occupancy(3) > occupancy(nbw) + 0.1)
            nbw = 3;
        // Above 16 rows (up to 64, or 128 over a weight of at most 16 MiB):
        // a CU's time goes with the bytes it requests (A rows plus weight
        // rows of its tiles, times its rounds of tiles), so take the 16-,
        // 32- or 64-row tile that needs the fewest.  Measured
        // on MI355X (us per call, old tile -> chosen tile): 32 x 6144 x 2048
        // 32 x 32 7.43 -> two 16 x 48 7.06; 48 x 4096 x 4096 64 x 16 12.19
        // -> two 32 x 32 9.95; 40 x 6144 x 2048 64 x 32 10.12 -> two 32 x 64
        // 8.66; 48 x 2048 x 4096 64 x 16 9.00 -> three 16 x 32 7.33; the
        // other candidates in the model's order.  Weights of 48 MiB and
        // more with up to 32 rows go to the ring kernel below, which keeps
        // 32-row blocks.
        bool by_cost = false;
        if (m > 16 && wbytes < (48ull << 20)) {
            if (stream_tile_cost(m, nb16, p.cu_count, st16.mb, st16.nb) <
                stream_tile_cost(m, nb16, p.cu_count, p.m_blocks, nbw)) {
                p.m_blocks = st16.mb;
                nbw = st16.nb;
            }
            m_tiles = div_up(m, 16 * p.m_blocks);
            by_cost = true;
            why = "small m: stream kernel, the tile asking each CU for the fewest A and weight "
                  "bytes";
        }
        p.n_blocks = nbw;
        const uint32_t pairs = p.m_blocks * p.n_blocks;
        p.waves = pairs == 1 ? 16 : (pairs <= 4 ? 8 : 4);
        // 32 x 64 tiles: 8 waves measured 7-8 % faster than 4 (40 x 6144 x
        // 2048: 8.66 vs 9.35 us; 64 x 6144 x 2048: 9.30 vs 9.93 us).
        if (by_cost && p.m_blocks == 2 && p.n_blocks == 4)
            p.waves = 8;
        while (p.waves > 4 && ksteps < 2 * p.waves)
            p.waves /= 2;
        const uint32_t tiles = div_up(nb16, nbw) * m_tiles;
        // Split K only when the tiles would leave most CUs idle.  Splits
        // publish their partials with write-through stores, never with a
        // release fence (a device-scope release of a split partial measured
        // 40-90 us per call over such grids).  Splits double while the grid
        // fits the CUs, each split keeps 8 or more K steps and every XCD's
        // range of the grid holds whole tiles (a tile's splits share one
        // XCD); a
        // split of 32 or more steps keeps 16 waves, shorter ones take 8
        // (measured on MI355X, us per call: 1 x 1024 x 8192 48.9 -> 5.6,
        // 16 x 1024 x 8192 50.1 -> 6.2, 4 x 2048 x 14336 95.2 -> 8.6,
        // 8 x 512 x 8192 7.4 unsplit -> 5.4).
        auto xcd_whole = [&](uint32_t sp) {
            const uint32_t grid = tiles * sp;
            return grid % 8 == 0 && (grid / 8) % sp == 0;
        };
        p.splits = 1;
        if (tiles * 2 <= p.cu_count) {
            while (tiles * p.splits * 2 <= p.cu_count && ksteps / (p.splits * 2) >= 8 &&
                   xcd_whole(p.splits * 2))
                p.splits *= 2;
        }
        if (p.splits > 1) {
            p.flags |= W8A16_FLAG_XCD_LOCAL;
            const uint32_t sps = div_up(ksteps, p.splits);
            const uint32_t wmax = sps >= 32 ? 16u : 8u;
            if (p.waves > wmax)
                p.waves = wmax;
        }

        // A large weight (>= 48 MiB) with 8..32 rows streams faster through
        // the ring kernel's row-contiguous LDS-DMA stages (measured 3-9 %);
        // below that, or with fewer rows, its slower start does not pay off.
        const uint32_t rmb = m <= 16 ? 1 : 2;
        if (m >= 8 && m <= 32 && wbytes >= (48ull << 20) && p.splits == 1 && nbw != 3) {
            const bool a8 = m <= 8;
            // 16 waves measured best for 16 rows x 64 columns, else 8; three
            // stages in flight unless LDS allows only two.
            const uint32_t wcand[2] = {(rmb == 1 && nbw == 4) ? 16u : 8u,
                                       (rmb == 1 && nbw == 4) ? 8u : 16u};
            bool chosen = false;
            for (uint32_t wi = 0; wi < 2 && !chosen; ++wi) {
                for (uint32_t depth = 3; depth >= 2 && !chosen; --depth) {
                    const uint32_t rw = wcand[wi];
                    if (!ring_shape_ok(rmb, nbw, 4, depth, rw, a8) || ksteps > rw * 64u ||
                        ring_lds_bytes(rmb, nbw, 4, depth, a8, ksteps) > kMaxLdsBytes)
                        continue;
                    p.kernel = W8A16_KERNEL_RING;
                    p.m_blocks = rmb;
                    p.n_blocks = nbw;
                    p.stage_steps = 4;
                    p.depth = depth;
                    p.waves = rw;
                    chosen = true;
                    why = "8..32 rows over a weight of 48 MiB or more: ring kernel";
                }
            }
        }
    }
    st = plan_finalize(m, n, k, &p);
    if (st != W8A16_OK)
        return st;
    if (p.splits > 1)
        set_reason("%s; K split %u ways (%u tiles for %u CUs)", why, p.splits,
                   p.m_tiles * p.n_tiles, p.cu_count);
    else
        set_reason("%s", why);
    *out = p;
    return W8A16_OK;
}

int check_args_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t a_row_stride,
                    uint32_t c_row_stride)
{
    // m, k and both pitches as the W8A16 GEMM checks them; the A pitch in
    // FP4 elements must keep rows 16-byte aligned (a multiple of 32)
    int st = check_args(m, n, k, a_row_stride, c_row_stride);
    if (st == W8A16_ERR_A_STRIDE_ALIGN || (st == W8A16_OK && a_row_stride % 32 != 0)) {
        char buf[160];
        snprintf(buf, sizeof buf,
                 "w8a16_gemm_w4a4: a_row_stride=%u must keep FP4 rows 16B-aligned "
                 "(multiple of 32 elements)", a_row_stride);
        return fail(W8A16_ERR_A_STRIDE_ALIGN, buf);
    }
    if (st != W8A16_OK)
        return fail_with_name(st, "w8a16_gemm_w4a4");
    // the kernels address a tile's rows (at most 64) through 32-bit buffer
    // ranges below 2^31 bytes
    if (k > kW4a4MaxK || a_row_stride > kW4a4MaxK) {
        char buf[160];
        snprintf(buf, sizeof buf,
                 "w8a16_gemm_w4a4: k=%u and a_row_stride=%u must be at most %u elements", k,
                 a_row_stride, kW4a4MaxK);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    return W8A16_OK;
}

// The page's tiers (m <= 8, 9..16, 17..32, 33..64) choose how many 16-row
// weight tiles share each activation fragment (1, 2, 4, 2) and send 9..32
// rows over a wide weight to the persistent entry.  Re-derived for MI355X,
// where a CU streams at most about 20 KiB/us from HBM, so every CU must get
// an equal share of the weight and A must not be re-read per tile: the
// persistent kernel (A once per CU in LDS, equal contiguous tile ranges per
// CU, K split over the waves) when the weight has two or more 16-row tiles
// per CU and A fits in LDS; otherwise (a weight of one tile per CU or so is
// read in one round trip, and the tiled kernel starts it sooner) the tile
// (16, 32 or 64 rows by 16, 32 or 64 columns) whose rounds of tiles ask
// each CU for the fewest FP4 bytes of A and weight rows per K (the W8A16
// stream planner's rule), ties to fewer blocks per tile.
int make_plan_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out)
{
    if (!out)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_plan: null plan");
    int st = check_args_w4a4(m, n, k, k, n);
    if (st != W8A16_OK)
        return st;
    char buf[128];
    if (m > kW4a4MaxM) {
        snprintf(buf, sizeof buf, "w8a16_gemm_w4a4: m=%u exceeds the W4A4 tiers' %u rows", m,
                 kW4a4MaxM);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    w8a16_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.cu_count = cu_count ? cu_count : kDefaultCUs;
    p.splits = 1;
    const uint32_t ksteps = k / kKStep;
    const uint32_t n16 = div_up(n, 16);
    // persistent kernel when the weight has at least kW4a4PsMinTilesPerCu
    // 16-row tiles per CU and A fits in LDS: 8 waves (measured ahead of 16
    // on MI355X), 4 when the workgroup has fewer items (tiles x groups of 4
    // K steps) or LDS room
    const uint32_t ps_mb = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    const uint32_t ps_grid = p.cu_count < n16 ? p.cu_count : n16;
    const uint64_t ps_items = (uint64_t)div_up(n16, ps_grid) * div_up(ksteps, 4);
    uint32_t ps_waves = 8;
    if (w4a4_ps_lds_bytes(ps_mb, k, ps_waves) > kMaxLdsBytes || ps_items < ps_waves)
        ps_waves = 4;
    if (n16 >= kW4a4PsMinTilesPerCu * p.cu_count &&
        w4a4_ps_lds_bytes(ps_mb, k, ps_waves) <= kMaxLdsBytes) {
        p.kernel = W8A16_KERNEL_W4A4_PS;
        p.m_blocks = ps_mb;
        p.n_blocks = 1;
        p.waves = ps_waves;
        set_reason("W4A4: %u or more 16-row weight tiles per CU and A fits in LDS: "
                   "persistent kernel", kW4a4PsMinTilesPerCu);
    } else {
        p.kernel = W8A16_KERNEL_W4A4;
        uint64_t best = ~0ull;
        const uint32_t opts[3] = {1, 2, 4};
        for (uint32_t mb : opts)
            for (uint32_t nb : opts) {
                if (!w4a4_shape_supported(mb, nb))
                    continue;
                const uint64_t tiles = (uint64_t)div_up(m, 16 * mb) * div_up(n16, nb);
                const uint64_t cost = (tiles + p.cu_count - 1) / p.cu_count * (mb + nb);
                if (cost < best || (cost == best && mb * nb < p.m_blocks * p.n_blocks)) {
                    best = cost;
                    p.m_blocks = mb;
                    p.n_blocks = nb;
                }
            }
        // the most waves whose registers hold two groups of 4 steps, fewer
        // until every wave has two groups
        p.waves = w4a4_variant_ok(p.m_blocks, p.n_blocks, 16) ? 16
                  : (w4a4_variant_ok(p.m_blocks, p.n_blocks, 8) ? 8 : 4);
        const uint32_t groups = div_up(ksteps, 4);
        while (p.waves > 4 && groups < 2 * p.waves)
            p.waves /= 2;
        set_reason("W4A4: tiled kernel, the tile asking each CU for the fewest bytes");
    }
    st = plan_finalize(m, n, k, &p);
    if (st != W8A16_OK)
        return st;
    *out = p;
    return W8A16_OK;
}

const char *status_string(int status)
{
    switch (status) {
    case W8A16_OK: return "ok";
    case W8A16_ERR_M_ZERO: return "m must be >= 1";
    case W8A16_ERR_K_NOT_MULT_128: return "k must be a positive multiple of 128";
    case W8A16_ERR_PITCH_TOO_SHORT: return "row pitch shorter than the used extent";
    case W8A16_ERR_A_STRIDE_ALIGN: return "a_row_stride must be a multiple of 8";
    case W8A16_ERR_N_ZERO: return "n must be >= 1";
    case W8A16_ERR_NULL_PTR: return "null pointer argument";
    case W8A16_ERR_BAD_PLAN: return "plan does not fit the problem";
    case W8A16_ERR_HIP: return "HIP runtime error";
    case W8A16_ERR_WORKSPACE: return "split-K workspace unavailable (growth during capture, "
                                     "or beyond the no-alloc scratch)";
    case W8A16_ERR_ENV: return "W8A16_LOG or W8A16_DEBUG_SYNC is set to a value other than 0 or 1";
    default: return "unknown status";
    }
}

int make_plan_w8a8(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out)
{
    if (!out)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_plan: null plan");
    int st = check_args(m, n, k, k, n);
    if (st != W8A16_OK)
        return st;
    // The stream kernel's small-m rule: 16-row blocks covering up to 64
    // rows (taller m takes several row tiles), the widest column tile that
    // still gives about three quarters of the CUs a tile, at least two K
    // steps per wave.  No K split.
    w8a16_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.cu_count = cu_count ? cu_count : kDefaultCUs;
    p.kernel = W8A16_KERNEL_W8A8;
    p.m_blocks = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    p.splits = 1;
    const uint32_t ksteps = k / kKStep;
    uint32_t m_tiles = div_up(m, 16 * p.m_blocks);
    const uint32_t fill = (3 * p.cu_count) / 4;
    p.n_blocks = 1;
    const uint32_t cands[3] = {4, 2, 1};
    for (uint32_t c : cands)
        if (w8a8_shape_supported(p.m_blocks, c) && div_up(n, 16 * c) * m_tiles >= fill) {
            p.n_blocks = c;
            break;
        }
    // 48-column tiles when they fill the CUs' last round of tiles clearly
    // better (as for the stream kernel).
    auto occupancy = [&](uint32_t c) {
        const uint64_t t = (uint64_t)div_up(n, 16 * c) * m_tiles;
        const uint64_t rounds = (t + p.cu_count - 1) / p.cu_count;
        return (double)t / (double)(rounds * p.cu_count);
    };
    if (w8a8_shape_supported(p.m_blocks, 3) && p.n_blocks > 1 &&
        occupancy(3) > occupancy(p.n_blocks) + 0.1)
        p.n_blocks = 3;
    // Above 16 rows, the tile that asks each CU for the fewest bytes: its
    // FP8 A rows plus weight rows, times its rounds of tiles; ties go to
    // fewer rows.  Measured on MI355X (us per call, old tile -> chosen):
    // 48 x 4096 x 4096 64 x 16 11.13 -> two 32 x 32 8.76; 64 x 4096 x 4096
    // 12.29 -> 9.54; 40 x 6144 x 2048 64 x 32 8.16 -> 32 x 64 7.77;
    // 32 x 6144 x 2048 32 x 32 6.57 -> 16 x 48 6.45; 24 x 4096 x 4096
    // 32 x 16 7.04 -> 16 x 32 6.83.
    if (m > 16) {
        const uint32_t nb16 = div_up(n, 16);
        auto cost = [&](uint32_t mb, uint32_t nb) {
            const uint64_t t = (uint64_t)div_up(m, 16 * mb) * div_up(nb16, nb);
            return (t + p.cu_count - 1) / p.cu_count * (16ull * mb + 16ull * nb);
        };
        uint64_t best = ~0ull;
        uint32_t bmb = p.m_blocks, bnb = p.n_blocks;
        const uint32_t mbs[3] = {1, 2, 4}, nbs[4] = {4, 3, 2, 1};
        for (uint32_t mb : mbs)
            for (uint32_t nb : nbs)
                if (w8a8_shape_supported(mb, nb) && cost(mb, nb) < best) {
                    best = cost(mb, nb);
                    bmb = mb;
                    bnb = nb;
                }
        if (best <= cost(p.m_blocks, p.n_blocks)) {
            p.m_blocks = bmb;
            p.n_blocks = bnb;
            m_tiles = div_up(m, 16 * p.m_blocks);
        }
    }
    // Eight waves up to four blocks per tile (each keeps two K steps in
    // flight; sixteen measured 5 % slower at 8 x 4096 x 4096), else four.
    const uint32_t pairs = p.m_blocks * p.n_blocks;
    set_reason("W8A8: widest column tile giving 3/4 of the CUs a tile%s",
               m > 16 ? ", or the one asking each CU for the fewest bytes" : "");
    p.waves = pairs <= 4 ? 8 : 4;
    while (p.waves > 4 && (ksteps < 2 * p.waves ||
                           w8a8_lds_bytes(p.m_blocks, p.n_blocks, p.waves) > kMaxLdsBytes))
        p.waves /= 2;
    st = plan_finalize(m, n, k, &p);
    if (st != W8A16_OK)
        return st;
    *out = p;
    return W8A16_OK;
}

// Replace the "w8a16_gemm" prefix of the thread's last error by `name`.
int fail_with_name(int status, const char *name)
{
    char buf[320];
    const char *msg = last_error();
    snprintf(buf, sizeof buf, "%s: %s", name,
             strncmp(msg, "w8a16_gemm: ", 12) == 0 ? msg + 12 : msg);
    return fail(status, buf);
}

// Prefix the thread's last error with the index of the descriptor it came
// from and return `status`.
int fail_at(int status, uint32_t index)
{
    char buf[320];
    const char *msg = last_error();
    snprintf(buf, sizeof buf, "w8a16_gemm_batched: descriptor %u: %s", index,
             strncmp(msg, "w8a16_gemm: ", 12) == 0 ? msg + 12 : msg);
    return fail(status, buf);
}

int plan_batched(const w8a16_gemm_desc_t *descs, uint32_t count, uint32_t cu_count,
                 w8a16_plan_t *out)
{
    char buf[256];
    if (!descs || !out)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_gemm_batched: null descriptors or plan");
    if (count < 1 || count > W8A16_MAX_BATCH) {
        snprintf(buf, sizeof buf, "w8a16_gemm_batched: count=%u must be in 1..%u", count,
                 (unsigned)W8A16_MAX_BATCH);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    uint32_t max_m = 0, min_ksteps = 0xffffffffu;
    for (uint32_t i = 0; i < count; ++i) {
        const w8a16_gemm_desc_t &d = descs[i];
        int st = check_args(d.m, d.n, d.k, d.k, d.n);
        if (st != W8A16_OK)
            return fail_at(st, i);
        if (d.m > 64) {
            snprintf(buf, sizeof buf,
                     "w8a16_gemm_batched: descriptor %u: m=%u exceeds the batched tier's 64 rows",
                     i, d.m);
            return fail(W8A16_ERR_BAD_PLAN, buf);
        }
        max_m = d.m > max_m ? d.m : max_m;
        min_ksteps = d.k / kKStep < min_ksteps ? d.k / kKStep : min_ksteps;
    }
    // One stream-kernel variant for all problems, chosen as the single-GEMM
    // rule chooses it for the tallest problem and the total column count:
    // 16-row blocks covering m, the widest column tile that still gives
    // about three quarters of the CUs a tile, waves by blocks per tile.
    w8a16_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.cu_count = cu_count ? cu_count : kDefaultCUs;
    p.kernel = W8A16_KERNEL_STREAM;
    p.m_blocks = max_m <= 16 ? 1 : (max_m <= 32 ? 2 : 4);
    p.depth = 1;
    p.splits = 1;
    const uint32_t fill = (3 * p.cu_count) / 4;
    auto tiles_for = [&](uint32_t nbw) {
        uint64_t t = 0;
        for (uint32_t i = 0; i < count; ++i)
            t += (uint64_t)div_up(descs[i].m, 16 * p.m_blocks) * div_up(descs[i].n, 16 * nbw);
        return t;
    };
    p.n_blocks = 1;
    const uint32_t cands[3] = {4, 2, 1};
    for (uint32_t c : cands)
        if (stream_shape_supported(p.m_blocks, c) && tiles_for(c) >= fill) {
            p.n_blocks = c;
            break;
        }
    // Above 16 rows, the single-GEMM bytes-per-CU choice over all arms'
    // tiles: the 16-, 32- or 64-row tile whose rounds of tiles ask each CU
    // for the fewest A and weight bytes (32 x 128 tiles left out).
    bool by_cost = false;
    if (max_m > 16) {
        const uint32_t keep_mb = p.m_blocks, keep_nb = p.n_blocks;
        auto cost = [&](uint32_t mb, uint32_t nb) {
            p.m_blocks = mb;
            const uint64_t t = tiles_for(nb);
            return (t + p.cu_count - 1) / p.cu_count * (32ull * mb + 16ull * nb);
        };
        uint64_t best = cost(keep_mb, keep_nb);
        uint32_t bmb = keep_mb, bnb = keep_nb;
        const uint32_t mbs[3] = {4, 2, 1}, nbs[5] = {8, 4, 3, 2, 1};
        for (uint32_t mb : mbs)
            for (uint32_t nb : nbs) {
                if (!stream_shape_supported(mb, nb) || (mb == 2 && nb == 8))
                    continue;
                const uint64_t c = cost(mb, nb);
                if (c < best) {
                    best = c;
                    bmb = mb;
                    bnb = nb;
                }
            }
        p.m_blocks = bmb;
        p.n_blocks = bnb;
        by_cost = true;
    }
    const uint32_t pairs = p.m_blocks * p.n_blocks;
    p.waves = pairs == 1 ? 16 : (pairs <= 4 ? 8 : 4);
    if (by_cost && p.m_blocks == 2 && p.n_blocks == 4)
        p.waves = 8;
    while (p.waves > 4 && min_ksteps < 2 * p.waves)
        p.waves /= 2;
    // Finalize against the tallest, widest, longest problem for the block,
    // LDS and variant checks; then describe the whole grid.
    uint32_t max_n = 0, max_k = 0;
    for (uint32_t i = 0; i < count; ++i) {
        max_n = descs[i].n > max_n ? descs[i].n : max_n;
        max_k = descs[i].k > max_k ? descs[i].k : max_k;
    }
    int st = plan_finalize(max_m, max_n, max_k, &p);
    if (st != W8A16_OK)
        return st;
    const uint64_t grid = tiles_for(p.n_blocks);
    if (grid > 0x7fffffffull)
        return fail(W8A16_ERR_BAD_PLAN, "w8a16_gemm_batched: grid too large");
    p.grid = (uint32_t)grid;
    p.m_tiles = div_up(max_m, 16 * p.m_blocks);
    p.n_tiles = 0;
    for (uint32_t i = 0; i < count; ++i)
        p.n_tiles += div_up(descs[i].n, 16 * p.n_blocks);
    p.steps_per_split = max_k / kKStep;
    set_reason("batched: one stream-kernel tile for all %u problems, chosen for the tallest", count);
    *out = p;
    return W8A16_OK;
}

}  // namespace w8a16

extern "C" {

int w8a16_plan_w8a8(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out)
{
    return w8a16::make_plan_w8a8(m, n, k, cu_count, out);
}

int w8a16_plan_w4a4(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out)
{
    return w8a16::make_plan_w4a4(m, n, k, cu_count, out);
}

int w8a16_plan_batched(const w8a16_gemm_desc_t *descs, uint32_t count, uint32_t cu_count,
                       w8a16_plan_t *out)
{
    return w8a16::plan_batched(descs, count, cu_count, out);
}

int w8a16_check_args(uint32_t m, uint32_t n, uint32_t k, uint32_t a_row_stride,
                     uint32_t c_row_stride)
{
    return w8a16::check_args(m, n, k, a_row_stride, c_row_stride);
}

int w8a16_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out)
{
    return w8a16::make_plan(m, n, k, cu_count, out);
}

int w8a16_plan_finalize(uint32_t m, uint32_t n, uint32_t k, w8a16_plan_t *plan)
{
    return w8a16::plan_finalize(m, n, k, plan);
}

const char *w8a16_status_string(int status) { return w8a16::status_string(status); }

const char *w8a16_last_error(void) { return w8a16::last_error(); }

}  // extern "C"
