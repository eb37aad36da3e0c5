// gemm_dma_shared.hip -- instantiation of the direct-to-LDS GEMM engine for the shared experts'
// gate/up with SiTU (one unit per kind, so the units compile in parallel).
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma<EPI_SITU, true, false, uint16_t, false>(int, const GemmArgs &,
                                                                       hipStream_t);

}  // namespace moe
