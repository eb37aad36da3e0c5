// gemm_dma_bwd_nt.hip -- instantiation of the direct-to-LDS GEMM engine for the backward pass's
// recomputed pre-activations with fp32 output: dense, and grouped with gathered A rows.
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma<EPI_STORE, false, false, float, false>(int, const GemmArgs &,
                                                                      hipStream_t);
template hipError_t launch_dma<EPI_STORE, false, true, float, false>(int, const GemmArgs &,
                                                                     hipStream_t);

}  // namespace moe
