// gemm_dma_mx4.hip -- instantiation of the direct-to-LDS GEMM engine for the
// routed experts' GEMMs with MXFP4 weights (gate/up with the SiTU epilogue,
// and down), with bf16 activations and with MX FP8 activations.
#include "gemm_launch.h"

namespace moe {

template hipError_t launch_dma_b4<EPI_STORE, false, false, uint16_t>(int, const GemmArgs &,
                                                                    hipStream_t);
template hipError_t launch_dma_b4<EPI_SITU, true, true, uint16_t>(int, const GemmArgs &,
                                                                 hipStream_t);

template hipError_t launch_dma_b4a8<EPI_STORE, false, false, uint16_t>(int, const GemmArgs &,
                                                                     hipStream_t);
template hipError_t launch_dma_b4a8<EPI_SITU, true, true, uint16_t>(int, const GemmArgs &,
                                                                  hipStream_t);

}  // namespace moe
