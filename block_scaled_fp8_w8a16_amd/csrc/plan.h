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
constexpr uint32_t kTileThreads = 256;           // tile kernel: 4 waves
constexpr uint32_t kTileRows = 128;              // tile kernel: rows of C per tile
constexpr uint32_t kTileMaxSteps = 64;           // tile kernel: K steps per split (one per lane)

// LDS of the tile kernel for a 128 x (16 * n_blocks) C tile: two buffers of
// one K step of A (128 rows x 256 bytes of BF16) and `stages` buffers of one
// K step of the FP8 weight (16 * n_blocks rows x 128 bytes).
constexpr uint32_t tile_lds_bytes(uint32_t n_blocks, uint32_t stages)
{
    return 2 * kTileRows * 256 + stages * 16 * n_blocks * 128;
}

int check_args(uint32_t m, uint32_t n, uint32_t k, uint32_t a_row_stride,
               uint32_t c_row_stride);
int make_plan(uint32_t m, uint32_t n, uint32_t k, uint32_t cu_count, w8a16_plan_t *out);
int plan_finalize(uint32_t m, uint32_t n, uint32_t k, w8a16_plan_t *p);
const char *status_string(int status);
const char *last_error();
void set_last_error(const char *msg);
int fail(int status, const char *msg);

}  // namespace w8a16
