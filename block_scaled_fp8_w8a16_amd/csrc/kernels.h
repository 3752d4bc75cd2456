// Kernel launch interface shared by the C ABI and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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

// W4A4 MX GEMV operands: packed FP4 (two E2M1 per byte, even element in the
// low nibble) with one E8M0 scale byte per 32 K elements of a row.
struct MxArgs {
    const uint8_t *a;       // FP4 [m, a_stride bytes]
    const uint8_t *a_scale; // E8M0 [m, k/32]
    const uint8_t *w;       // FP4 [n, k/2 bytes]
    const uint8_t *w_scale; // E8M0 [n, k/32]
    uint8_t *c;             // BF16 [m, c_stride]
    uint32_t a_stride;      // A row pitch in bytes
    uint32_t c_stride, m, n, k, m_tiles, n_tiles;
    // persistent kernel: workgroup g owns tiles_base + (g < tiles_extra)
    // 16-row weight tiles, starting at g * tiles_base + min(g, tiles_extra)
    uint32_t tiles_base, tiles_extra;
};

// FP8 activation quantizer: A BF16 [m, a_stride] -> codes [m, q_stride] and
// scales [m, k/128].
struct QuantArgs {
    const uint8_t *a;
    uint8_t *q;
    float *scales;
    uint32_t a_stride, q_stride, m, k;
};

// A launch of `kern` needs `bytes` of dynamic LDS: above the 64 KiB
// default, raise the kernel's limit to `limit` (the most any plan uses) on
// the current device.  The attribute is per device, so it is set once per
// device id (bit i of `done`; ids of 64 and above are set on every call).
inline hipError_t allow_lds(const void *kern, uint32_t bytes, uint32_t limit,
                            std::atomic<uint64_t> &done)
{
    if (bytes <= 65536)
        return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(limit > bytes ? limit : bytes));
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

hipError_t launch_stream(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_act_quant(const QuantArgs &q, hipStream_t stream);
// W8A8: g.a holds FP8 codes (g.a_stride in bytes), a_scales FP32 [m, k/128].
hipError_t launch_w8a8(const GemmArgs &g, const float *a_scales, const w8a16_plan_t &p,
                       hipStream_t stream);
hipError_t launch_stream_batched(const BatchArgs &b, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_w4a4(const MxArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_tile_m64(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_tile_m128(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
hipError_t launch_ring(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
// 128 x 256 tiles (tile plans with m_blocks 8, n_blocks 16).
hipError_t launch_wide(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream);
// Adds the K splits of a tile plan's workspace ([splits][ws_rows][ws_cols]
// FP32, whole tiles) in split order and stores C.
hipError_t launch_split_reduce(const GemmArgs &g, uint32_t ws_cols, uint32_t ws_rows,
                               hipStream_t stream);

}  // namespace w8a16
