// Host-only driver for the planner (plan.cpp), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by the CPU test suite.  It calls every pure
// entry point of the boundary -- w8a16_check_args, w8a16_plan,
// w8a16_plan_w8a8, w8a16_plan_w4a4, w8a16_plan_batched,
// w8a16_plan_finalize, w8a16_status_string, w8a16_last_error -- over a
// sweep of shapes (1 row to the largest, K up to 2^24, every CU count the
// planner takes) and over caller-edited plans whose fields are drawn at
// random, including values far outside what the kernels support.  A
// sanitizer report aborts the run; an accepted plan that does not cover its
// problem or does not fit a compute unit's LDS exits with status 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "w8a16.h"

namespace {

uint64_t g_state = 0x243f6a8885a308d3ull;

// xorshift64 (Marsaglia, "Xorshift RNGs", 2003)
uint32_t next_u32()
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 32);
}

// A descriptor field: usually small, sometimes zero or anything.
uint32_t wild(uint32_t small)
{
    const uint32_t r = next_u32();
    if (r % 8 == 0)
        return next_u32();
    if (r % 8 == 1)
        return 0;
    return next_u32() % (small + 1);
}

int g_fail = 0;
unsigned long g_accepted = 0, g_rejected = 0;

void expect(bool ok, const char *what, uint32_t m, uint32_t n, uint32_t k, const w8a16_plan_t &p)
{
    if (ok)
        return;
    std::fprintf(stderr,
                 "%s: m=%u n=%u k=%u kernel=%u mb=%u nb=%u splits=%u steps=%u tiles=%ux%u "
                 "grid=%u block=%u lds=%u\n",
                 what, m, n, k, p.kernel, p.m_blocks, p.n_blocks, p.splits, p.steps_per_split,
                 p.m_tiles, p.n_tiles, p.grid, p.block, p.lds_bytes);
    g_fail = 1;
}

// Invariants of any accepted plan of the W8A16 / W8A8 kernels.
void check_plan(uint32_t m, uint32_t n, uint32_t k, const w8a16_plan_t &p)
{
    const uint32_t ksteps = k / 128;
    expect(p.grid >= 1 && p.block >= 64 && p.block <= 1024 && p.block % 64 == 0,
           "launch shape", m, n, k, p);
    expect(p.lds_bytes <= 160 * 1024, "LDS above 160 KiB", m, n, k, p);
    expect(p.splits >= 1 && p.steps_per_split >= 1 &&
               (uint64_t)p.splits * p.steps_per_split >= ksteps &&
               (uint64_t)(p.splits - 1) * p.steps_per_split < ksteps,
           "K split does not cover K exactly", m, n, k, p);
    expect((uint64_t)p.m_tiles * 16 * p.m_blocks >= m &&
               (uint64_t)p.n_tiles * 16 * p.n_blocks >= n,
           "tiles do not cover C", m, n, k, p);
    expect(p.splits == 1 || p.workspace_bytes > 0, "split without workspace", m, n, k, p);
}

void check_w4a4_plan(uint32_t m, uint32_t n, uint32_t k, const w8a16_plan_t &p)
{
    expect(p.grid >= 1 && p.block >= 64 && p.block <= 1024 && p.lds_bytes <= 160 * 1024,
           "W4A4 launch shape", m, n, k, p);
    expect(p.kernel == W8A16_KERNEL_W4A4 || p.kernel == W8A16_KERNEL_W4A4_PS,
           "W4A4 kernel id", m, n, k, p);
    expect(16ull * p.m_blocks * (p.kernel == W8A16_KERNEL_W4A4 ? p.m_tiles : 1) >= m,
           "W4A4 rows not covered", m, n, k, p);
    expect(p.kernel == W8A16_KERNEL_W4A4_PS || (uint64_t)p.n_tiles * 16 * p.n_blocks >= n,
           "W4A4 columns not covered", m, n, k, p);
}

void touch_error()
{
    const char *e = w8a16_last_error();
    volatile size_t len = std::strlen(e);  // reads the whole message
    (void)len;
}

}  // namespace

int main()
{
    static const uint32_t ms[] = {1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65,
                                  96, 127, 128, 129, 200, 256, 511, 4096, 0};
    static const uint32_t ns[] = {1, 15, 16, 17, 128, 129, 1000, 2048, 4096, 6144,
                                  12288, 32768, 65535, 1u << 20, 0};
    static const uint32_t ks[] = {128, 256, 384, 2048, 4096, 5120, 8192, 65536,
                                  1u << 24, 100, 0};
    static const uint32_t cus[] = {0, 1, 8, 80, 256, 304, 1024};
    w8a16_plan_t p;

    for (int s = -3; s < 16; ++s)
        (void)std::strlen(w8a16_status_string(s));

    for (uint32_t m : ms)
        for (uint32_t n : ns)
            for (uint32_t k : ks)
                for (uint32_t cu : cus) {
                    std::memset(&p, 0xa5, sizeof p);
                    if (w8a16_plan(m, n, k, cu, &p) == W8A16_OK) {
                        check_plan(m, n, k, p);
                        w8a16_plan_t q = p;
                        expect(w8a16_plan_finalize(m, n, k, &q) == W8A16_OK &&
                                   std::memcmp(&p, &q, sizeof p) == 0,
                               "default plan is not a fixed point of finalize", m, n, k, p);
                    } else {
                        touch_error();
                    }
                    std::memset(&p, 0x5a, sizeof p);
                    if (w8a16_plan_w8a8(m, n, k, cu, &p) == W8A16_OK)
                        check_plan(m, n, k, p);
                    else
                        touch_error();
                    for (uint32_t k4 : {k, k / 4, k + 32}) {
                        std::memset(&p, 0x3c, sizeof p);
                        if (w8a16_plan_w4a4(m, n, k4, cu, &p) == W8A16_OK)
                            check_w4a4_plan(m, n, k4, p);
                        else
                            touch_error();
                    }
                    (void)w8a16_check_args(m, n, k, k + m, n + 8);
                    touch_error();
                }
    (void)w8a16_plan(1, 1, 128, 0, nullptr);
    touch_error();

    // Caller-edited plans, checked by finalize exactly as the planned entry
    // points do: a default plan with one to three fields changed to values
    // near the supported ones (now and then to any 32-bit value), on every
    // kernel id and one past the last.
    static const uint32_t waves_set[] = {0, 1, 2, 4, 6, 8, 10, 12, 16, 32};
    for (int it = 0; it < 400000; ++it) {
        const uint32_t m = 1 + next_u32() % (it % 3 == 0 ? 4096 : 160);
        const uint32_t n = 1 + next_u32() % 20000;
        const uint32_t k = 128 * (1 + next_u32() % 96) + (it % 97 == 0 ? 32 : 0);
        const uint32_t cu = next_u32() % 2 ? 256 : 1 + next_u32() % 300;
        std::memset(&p, 0, sizeof p);
        const uint32_t base = next_u32() % 3;
        const int st = base == 0   ? w8a16_plan(m, n, k, cu, &p)
                       : base == 1 ? w8a16_plan_w8a8(m, n, k, cu, &p)
                                   : w8a16_plan_w4a4(m, n, k, cu, &p);
        if (st != W8A16_OK) {
            touch_error();
            continue;
        }
        const uint32_t edits = 1 + next_u32() % 3;
        for (uint32_t e = 0; e < edits; ++e) {
            const uint32_t v = next_u32() % 16 == 0 ? next_u32() : next_u32() % 17;
            switch (next_u32() % 10) {
            case 0: p.kernel = next_u32() % 8; break;
            case 1: p.m_blocks = v % 9; break;
            case 2: p.n_blocks = v; break;
            case 3: p.splits = next_u32() % 4 == 0 ? v : 1 + next_u32() % 70; break;
            case 4: p.depth = v % 9; break;
            case 5: p.flags = v % 8; break;
            case 6: p.waves = waves_set[next_u32() % 10]; break;
            case 7: p.stage_steps = v % 10; break;
            case 8: p.a_depth = v % 8; break;
            default: p.cu_count = v == 0 ? 0 : next_u32() % 400; break;
            }
        }
        p.grid = next_u32();          // derived: finalize must overwrite these
        p.lds_bytes = next_u32();
        p.steps_per_split = next_u32();
        const bool w4 = p.kernel == W8A16_KERNEL_W4A4 || p.kernel == W8A16_KERNEL_W4A4_PS;
        if (w8a16_plan_finalize(m, n, k, &p) == W8A16_OK) {
            ++g_accepted;
            if (w4)
                check_w4a4_plan(m, n, k, p);
            else
                check_plan(m, n, k, p);
        } else {
            ++g_rejected;
            touch_error();
        }
    }

    // Batched plans from random descriptor lists, the count included.
    w8a16_gemm_desc_t d[W8A16_MAX_BATCH + 2];
    for (int it = 0; it < 20000; ++it) {
        const uint32_t count = next_u32() % (W8A16_MAX_BATCH + 2);
        for (uint32_t i = 0; i < count; ++i) {
            std::memset(&d[i], 0, sizeof d[i]);
            d[i].m = wild(80);
            d[i].n = 1 + next_u32() % 9000;
            d[i].k = 128 * (next_u32() % 40);
            d[i].a_row_stride = d[i].k;
            d[i].c_row_stride = d[i].n;
        }
        std::memset(&p, 0, sizeof p);
        if (w8a16_plan_batched(d, count, wild(300), &p) == W8A16_OK)
            expect(p.grid >= count && p.block % 64 == 0 && p.lds_bytes <= 160 * 1024,
                   "batched launch shape", d[0].m, d[0].n, d[0].k, p);
        else
            touch_error();
    }
    (void)w8a16_plan_batched(nullptr, 1, 0, &p);
    touch_error();

    std::printf("planner sweep done (%lu edited plans accepted, %lu rejected), %s\n",
                g_accepted, g_rejected, g_fail ? "INVARIANT FAILURES" : "ok");
    return g_fail;
}
