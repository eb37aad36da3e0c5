// gemm_dma_router.hip -- instantiation of the direct-to-LDS GEMM engine for router logits (fp32
// out) and the K-segmented output projection (one unit per kind, so the units compile in parallel).
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma<EPI_ROUTER, false, false, float, false>(int, const GemmArgs &,
                                                                       hipStream_t);
template hipError_t launch_dma<EPI_STORE, false, false, uint16_t, true>(int, const GemmArgs &,
                                                                       hipStream_t);

}  // namespace moe
