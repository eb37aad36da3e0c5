// activation.hip -- the SiTU-GLU factors evaluated elementwise on the device,
// through the same inline functions the GEMM epilogues call (common.h), so
// their numerics can be checked against fp64 over the whole input range.
//
// tech.news18a.com "KimiK3的StableLatentMoE架构解析", first technique: the
// sigmoid-limited, tanh-scaled unit whose output range is strictly bounded
// (beta = 4, beta_u = 25): phi(g) = sigmoid(g) beta tanh(g / beta),
// psi(u) = beta_u tanh(u / beta_u), h = phi(g) psi(u).
#include <algorithm>

#include "common.h"
#include "moe.h"

namespace moe {

__global__ void __launch_bounds__(256) situ_eval_kernel(const float *__restrict__ g,
                                                        const float *__restrict__ u, int64_t n,
                                                        float beta, float inv_beta, float beta_u,
                                                        float inv_beta_u,
                                                        float *__restrict__ phi,
                                                        float *__restrict__ psi,
                                                        float *__restrict__ h) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const float gi = g[i], ui = u[i];
    if (phi) phi[i] = situ_phi(gi, beta, inv_beta);
    if (psi) psi[i] = situ_psi(ui, beta_u, inv_beta_u);
    if (h) h[i] = situ(gi, ui, beta, inv_beta, beta_u, inv_beta_u);
  }
}

}  // namespace moe

MOE_API moe_status moe_situ_eval(const float *g, const float *u, int64_t n, float beta,
                                 float beta_u, float *phi, float *psi, float *h, void *stream) {
  if (n < 0 || !(beta > 0.0f) || !(beta_u > 0.0f)) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!g || !u || (!phi && !psi && !h)) return MOE_ERR_INVALID_ARG;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  if (moe::launch_kernel(moe::situ_eval_kernel, dim3((unsigned)blocks), dim3(256), 0,
                         static_cast<hipStream_t>(stream), g, u, n, beta, 1.0f / beta, beta_u,
                         1.0f / beta_u, phi, psi, h) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}
