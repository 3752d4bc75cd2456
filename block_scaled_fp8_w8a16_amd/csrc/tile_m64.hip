// The tile kernel's 64-row variants (m_blocks == 4).
#include "tile_kernel.h"

namespace w8a16 {

hipError_t launch_tile_m64(const GemmArgs &g, const w8a16_plan_t &p, hipStream_t stream)
{
    return launch_tile_rows<4>(g, p, stream);
}

}  // namespace w8a16
