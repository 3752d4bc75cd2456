// Fixed-order reduction of a tile plan's K splits (gfx950): C = the sum over
// splits, in split order, of the FP32 workspace tiles.  Shared by the tile
// and the wide tile kernels, which store whole FP32 tiles per split
// ([splits][ws_rows][ws_cols]); the kernel boundary publishes them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace w8a16 {

namespace {

using namespace dev;

// One thread per 4 adjacent outputs.
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

}  // namespace

hipError_t launch_split_reduce(const GemmArgs &g, uint32_t ws_cols, uint32_t ws_rows,
                               hipStream_t stream)
{
    const uint64_t threads = (uint64_t)g.m * (ws_cols / 4u);
    const uint32_t blocks = (uint32_t)((threads + 255u) / 256u);
    hipLaunchKernelGGL(w8a16_split_reduce_kernel, dim3(blocks), dim3(256), 0, stream, g, ws_cols,
                       ws_rows);
    return hipGetLastError();
}

}  // namespace w8a16
