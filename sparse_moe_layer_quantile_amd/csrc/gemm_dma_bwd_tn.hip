// gemm_dma_bwd_tn.hip -- instantiation of the direct-to-LDS GEMM engine for the backward pass's
// weight gradients: both operands K-outer (K = tokens or an expert's pairs), fp32 output; dense
// or one output per routed expert.
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma_ko<EPI_STORE, true, true, false, false, float>(int,
                                                                             const GemmArgs &,
                                                                             hipStream_t);
template hipError_t launch_dma_ko<EPI_STORE, true, true, true, false, float>(int,
                                                                            const GemmArgs &,
                                                                            hipStream_t);

}  // namespace moe
