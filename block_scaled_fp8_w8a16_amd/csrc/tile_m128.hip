// The tile kernel's 128-row variants (m_blocks == 8).
#include "tile_kernel.h"

namespace w8a16 {

hipError_t launch_tile_m128(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    return launch_tile_rows<8>(g, p, stream);
}

}  // namespace w8a16
