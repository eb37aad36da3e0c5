// gemm_dma_mx8.hip -- instantiation of the direct-to-LDS GEMM engine for the
// routed experts' GEMMs with MX FP8 weights and MX FP8 activations (gate/up
// with the SiTU epilogue, and down) on the block-scaled MFMA.
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma_b8a8<EPI_STORE, false, false, uint16_t>(int, const GemmArgs &,
                                                                     hipStream_t);
template hipError_t launch_dma_b8a8<EPI_SITU, true, true, uint16_t>(int, const GemmArgs &,
                                                                  hipStream_t);

}  // namespace moe
