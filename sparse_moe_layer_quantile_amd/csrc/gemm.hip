// gemm.hip -- instantiation and launch of the GEMM engine (see gemm.h).
#include "gemm.h"
#include "kernels.h"

namespace moe {

int gemm_bm(int path) { return path == PATH_F32 ? sf::BM : mf::BM; }
int gemm_bn_out(int path, bool dual) {
  const int bn = path == PATH_F32 ? sf::BN : mf::BN;
  return dual ? bn / 2 : bn;
}

template <int EPI, bool DUAL, bool FP8, bool GATHER, typename OutT>
static hipError_t launch_mfma(GemmArgs a, int64_t m_tiles, hipStream_t s) {
  const int bn_out = DUAL ? mf::BN / 2 : mf::BN;
  a.n_tiles_n = (int32_t)((a.N + bn_out - 1) / bn_out);
  const int64_t blocks = m_tiles * a.n_tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_mfma_kernel<EPI, DUAL, FP8, GATHER, OutT>), dim3((unsigned)blocks),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int EPI, bool DUAL, bool GATHER>
static hipError_t launch_f32(GemmArgs a, int64_t m_tiles, hipStream_t s) {
  const int bn_out = DUAL ? sf::BN / 2 : sf::BN;
  a.n_tiles_n = (int32_t)((a.N + bn_out - 1) / bn_out);
  const int64_t blocks = m_tiles * a.n_tiles_n;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI, DUAL, GATHER>), dim3((unsigned)blocks), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

// The contractions of the layer, by kind.
hipError_t gemm_launch(const GemmArgs &a, int path, GemmKind kind, bool fp8, int64_t m_tiles,
                       hipStream_t s) {
  if (path == PATH_F32) {
    switch (kind) {
      case GK_ROUTER: return launch_f32<EPI_ROUTER, false, false>(a, m_tiles, s);
      case GK_DENSE: return launch_f32<EPI_STORE, false, false>(a, m_tiles, s);
      case GK_DENSE_SITU: return launch_f32<EPI_SITU, true, false>(a, m_tiles, s);
      case GK_EXPERT_SITU: return launch_f32<EPI_SITU, true, true>(a, m_tiles, s);
      case GK_EXPERT_DOWN: return launch_f32<EPI_ROWSCALE, false, false>(a, m_tiles, s);
    }
    return hipErrorInvalidValue;
  }
  if (!fp8) {
    switch (kind) {
      case GK_ROUTER: return launch_mfma<EPI_ROUTER, false, false, false, float>(a, m_tiles, s);
      case GK_DENSE: return launch_mfma<EPI_STORE, false, false, false, uint16_t>(a, m_tiles, s);
      case GK_DENSE_SITU:
        return launch_mfma<EPI_SITU, true, false, false, uint16_t>(a, m_tiles, s);
      case GK_EXPERT_SITU:
        return launch_mfma<EPI_SITU, true, false, true, uint16_t>(a, m_tiles, s);
      case GK_EXPERT_DOWN:
        return launch_mfma<EPI_ROWSCALE, false, false, false, uint16_t>(a, m_tiles, s);
    }
  } else {
    switch (kind) {
      case GK_ROUTER: return hipErrorInvalidValue;  // the router stays bf16
      case GK_DENSE: return launch_mfma<EPI_STORE, false, true, false, uint16_t>(a, m_tiles, s);
      case GK_DENSE_SITU:
        return launch_mfma<EPI_SITU, true, true, false, uint16_t>(a, m_tiles, s);
      case GK_EXPERT_SITU:
        return launch_mfma<EPI_SITU, true, true, true, uint16_t>(a, m_tiles, s);
      case GK_EXPERT_DOWN:
        return launch_mfma<EPI_ROWSCALE, false, true, false, uint16_t>(a, m_tiles, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
