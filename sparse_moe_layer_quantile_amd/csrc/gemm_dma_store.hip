// gemm_dma_store.hip -- instantiation of the direct-to-LDS GEMM engine for dense W_down and the
// grouped expert down projection (one unit per kind, so the units compile in parallel).
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma<EPI_STORE, false, false, uint16_t, false>(int, const GemmArgs &,
                                                                       hipStream_t);

}  // namespace moe
