// gemm_dma_bwd_nn.hip -- instantiation of the direct-to-LDS GEMM engine for the backward pass's
// input gradients: the weight operand stored K-outer ([K][N], as the forward stores it), fp32
// output; dense or grouped, A rows as stored or gathered.
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma_ko<EPI_STORE, false, true, false, false, float>(int,
                                                                              const GemmArgs &,
                                                                              hipStream_t);
template hipError_t launch_dma_ko<EPI_STORE, false, true, false, true, float>(int,
                                                                             const GemmArgs &,
                                                                             hipStream_t);

}  // namespace moe
