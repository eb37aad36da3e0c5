// gemm_dma_fp8.hip -- instantiation of the direct-to-LDS GEMM engine for every single-segment GEMM
// with fp8 e4m3 weights (one unit per kind, so the units compile in parallel).
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma_b8<EPI_STORE, false, false, uint16_t, false>(int, const GemmArgs &,
                                                                           hipStream_t);
template hipError_t launch_dma_b8<EPI_STORE, false, false, uint16_t, true>(int, const GemmArgs &,
                                                                          hipStream_t);
template hipError_t launch_dma_b8<EPI_SITU, true, false, uint16_t, false>(int, const GemmArgs &,
                                                                   hipStream_t);
template hipError_t launch_dma_b8<EPI_SITU, true, true, uint16_t, false>(int, const GemmArgs &,
                                                                  hipStream_t);

}  // namespace moe
