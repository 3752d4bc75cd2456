// Kernel launch interface shared by the C ABI and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8a16.h"

namespace w8a16 {

constexpr uint32_t kWavesPerGroup = 4;

// Arguments every kernel takes (by value).  Pointers are device pointers;
// strides are in elements.
struct GemmArgs {
    const uint8_t *a;       // BF16 [m, a_stride]
    const uint8_t *w;       // E4M3 [n, k]
    const float *scale;     // FP32 [ceil(n/128), k/128]
    uint8_t *c;             // BF16 [m, c_stride]
    float *ws;              // split-K partial tiles (splits > 1)
    uint32_t *counters;     // split-K arrival counters, zero between calls
    uint32_t a_stride, c_stride, m, n, k;
    uint32_t m_tiles, n_tiles, splits, steps_per_split;
};

// Up to W8A16_MAX_BATCH GEMMs in one grid of the stream kernel: problem i
// owns logical workgroups start[i] .. start[i + 1] - 1 (start[0] == 0).
struct BatchArgs {
    GemmArgs g[W8A16_MAX_BATCH];
    uint32_t start[W8A16_MAX_BATCH];
    uint32_t count;
};

// FP8 activation quantizer: A BF16 [m, a_stride] -> codes [m, q_stride] and
// scales [m, k/128].
struct QuantArgs {
    const uint8_t *a;
    uint8_t *q;
    float *scales;
    uint32_t a_stride, q_stride, m, k;
};

hipError_t launch_stream(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_act_quant(const QuantArgs &q, hipStream_t stream);
// W8A8: g.a holds FP8 codes (g.a_stride in bytes), a_scales FP32 [m, k/128].
hipError_t launch_w8a8(const GemmArgs &g, const float *a_scales, const w8a16_plan_t &p,
                       hipStream_t stream);
hipError_t launch_stream_batched(const BatchArgs &b, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_tile_m64(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_tile_m128(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_ring(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);

}  // namespace w8a16
