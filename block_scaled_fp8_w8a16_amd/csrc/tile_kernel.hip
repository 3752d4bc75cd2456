// Tiled W8A16 GEMM kernel for large m (gfx950): not built yet; the planner
// never selects it.
#include "kernels.h"

namespace w8a16 {

hipError_t launch_tile(const GemmArgs &, const w8a16_plan_t &, hipStream_t)
{
    return hipErrorInvalidValue;
}

}  // namespace w8a16
