// gemm.hip -- dispatch of the layer's contractions to the GEMM engines (see
// gemm.h): tile shape per kind, the direct-to-LDS engine (gemm_dma_*.hip; bf16,
// fp8 and MXFP4 weights), the register-staged fp8 kernel for K ranges past the
// engine's scale table, fp32 SIMT.
#include <algorithm>
#include <cstdlib>

#include "gemm_launch.h"

namespace moe {

static_assert((int)WF_BF16 == g2::BF_BF16 && (int)WF_FP8 == g2::BF_FP8 &&
                  (int)WF_MX4 == g2::BF_MX4 && (int)WF_MX4A8 == g2::BF_MX4A8 &&
                  (int)WF_MX8A8 == g2::BF_MX8A8,
              "weight format codes");

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
  return launch_kernel(gemm_mfma_kernel<EPI, DUAL, FP8, GATHER, OutT>, dim3((unsigned)blocks),
                       dim3(256), 0, s, a);
}

template <int EPI, bool DUAL, bool GATHER>
static hipError_t launch_f32(GemmArgs a, int64_t m_tiles, hipStream_t s) {
  const int bn_out = DUAL ? sf::BN / 2 : sf::BN;
  a.n_tiles_n = (int32_t)((a.N + bn_out - 1) / bn_out);
  const int64_t blocks = m_tiles * a.n_tiles_n;
  if (blocks <= 0) return hipSuccess;
  return launch_kernel(gemm_f32_kernel<EPI, DUAL, GATHER>, dim3((unsigned)blocks), dim3(256), 0, s,
                       a);
}

// Tile shape of the bf16 engine per kind (a tuning override is read from
// MOE_GEMM_DENSE / MOE_GEMM_GROUPED).  Problems with a few rows (per expert)
// stream weights: they take a 32-row tile with a deep ring; otherwise grouped
// problems use 320 rows, which cover a typical expert in one M tile, and dense
// ones 256 x 256 tiles.
int dma_variant(GemmKind kind, int64_t rows, int64_t n_experts) {
  if (kind == GK_EXPERT_SITU || kind == GK_EXPERT_DOWN) {
    const int dflt = rows <= 8 * n_experts       ? kVSmallM
                     : rows <= 200 * n_experts ? kVGroupedShort
                                               : kVGrouped;
    const int v = env_int("MOE_GEMM_GROUPED", dflt);
    return bf16_shape(v) ? v : dflt;
  }
  const int dflt = rows <= 64 ? kVSmallM : kVDense;
  const int v = env_int("MOE_GEMM_DENSE", dflt);
  return bf16_shape(v) ? v : dflt;
}

int grouped_tile_rows(int path, int wf, int64_t rows, int64_t n_experts) {
  if (path == PATH_F32) return sf::BM;
  const int v = dma_variant(GK_EXPERT_SITU, rows, n_experts);
  // the MXFP4 engine's shapes (launch_dma_b4, launch_dma_b4a8)
  if (wf == WF_MX4A8) return kDma[a8_shape(rows, n_experts)].tm();
  if (wf == WF_MX8A8) return kDma[mx8_shape(rows, n_experts)].tm();
  if (wf == WF_MX4) return kDma[mx4_shape(v, rows, n_experts)].tm();
  // the fp8 engine's shapes (launch_dma_b8)
  if (wf == WF_FP8) return kDma[fp8_shape(v, true)].tm();
  return kDma[v].tm();
}

// The contractions of the layer, by kind.
hipError_t gemm_launch(const GemmArgs &a, int path, GemmKind kind, int wf, int64_t m_tiles,
                       hipStream_t s) {
  if (path == PATH_BF16 && wf == WF_MX4A8) {
    // MX FP8 activations x MXFP4 weights: the routed experts only
    const int v = a8_shape(a.M, a.n_experts);
    switch (kind) {
      case GK_EXPERT_SITU: return launch_dma_b4a8<EPI_SITU, true, true, uint16_t>(v, a, s);
      case GK_EXPERT_DOWN: return launch_dma_b4a8<EPI_STORE, false, false, uint16_t>(v, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (path == PATH_BF16 && wf == WF_MX8A8) {
    // MX FP8 activations x MX FP8 weights: the routed experts only
    const int v = mx8_shape(a.M, a.n_experts);
    switch (kind) {
      case GK_EXPERT_SITU: return launch_dma_b8a8<EPI_SITU, true, true, uint16_t>(v, a, s);
      case GK_EXPERT_DOWN: return launch_dma_b8a8<EPI_STORE, false, false, uint16_t>(v, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (path == PATH_BF16 && wf == WF_MX4) {
    // MXFP4 weights: the routed experts only
    const int v = mx4_shape(dma_variant(kind, a.M, a.n_experts), a.M, a.n_experts);
    switch (kind) {
      case GK_EXPERT_SITU: return launch_dma_b4<EPI_SITU, true, true, uint16_t>(v, a, s);
      case GK_EXPERT_DOWN: return launch_dma_b4<EPI_STORE, false, false, uint16_t>(v, a, s);
      default: return hipErrorInvalidValue;
    }
  }
  const bool fp8 = wf == WF_FP8;
  if (path == PATH_BF16 && !fp8) {
    const int v = dma_variant(kind, a.M, a.n_experts);
    switch (kind) {
      case GK_ROUTER: return launch_dma<EPI_ROUTER, false, false, float>(v, a, s);
      case GK_DENSE:
        if (a.nseg > 1) return launch_dma<EPI_STORE, false, false, uint16_t, true>(v, a, s);
        return launch_dma<EPI_STORE, false, false, uint16_t>(v, a, s);
      case GK_DENSE_SITU: return launch_dma<EPI_SITU, true, false, uint16_t>(v, a, s);
      case GK_EXPERT_SITU: return launch_dma<EPI_SITU, true, true, uint16_t>(v, a, s);
      case GK_EXPERT_DOWN: return launch_dma<EPI_STORE, false, false, uint16_t>(v, a, s);
    }
    return hipErrorInvalidValue;
  }
  if (path == PATH_F32) {
    switch (kind) {
      case GK_ROUTER: return launch_f32<EPI_ROUTER, false, false>(a, m_tiles, s);
      case GK_DENSE: return launch_f32<EPI_STORE, false, false>(a, m_tiles, s);
      case GK_DENSE_SITU: return launch_f32<EPI_SITU, true, false>(a, m_tiles, s);
      case GK_EXPERT_SITU: return launch_f32<EPI_SITU, true, true>(a, m_tiles, s);
      case GK_EXPERT_DOWN: return launch_f32<EPI_STORE, false, false>(a, m_tiles, s);
    }
    return hipErrorInvalidValue;
  }
  // fp8 e4m3 weights with block scales (bf16 activations): the direct-to-LDS
  // engine with the block scales of up to 128 K blocks staged in LDS; the
  // register-staged kernel beyond that
  int64_t kblocks = 0;
  for (int i = 0; i < a.nseg; ++i) kblocks += a.seg[i].k / 128;
  if (kblocks <= g2::kMaxKBlocks) {
    const bool grouped = kind == GK_EXPERT_SITU || kind == GK_EXPERT_DOWN;
    const int v = fp8_shape(dma_variant(kind, a.M, a.n_experts), grouped);
    switch (kind) {
      case GK_ROUTER: return hipErrorInvalidValue;  // the router stays bf16
      case GK_DENSE:
        if (a.nseg > 1) return launch_dma_b8<EPI_STORE, false, false, uint16_t, true>(v, a, s);
        return launch_dma_b8<EPI_STORE, false, false, uint16_t>(v, a, s);
      case GK_DENSE_SITU: return launch_dma_b8<EPI_SITU, true, false, uint16_t>(v, a, s);
      case GK_EXPERT_SITU: return launch_dma_b8<EPI_SITU, true, true, uint16_t>(v, a, s);
      case GK_EXPERT_DOWN: return launch_dma_b8<EPI_STORE, false, false, uint16_t>(v, a, s);
    }
    return hipErrorInvalidValue;
  }
  switch (kind) {
    case GK_ROUTER: return hipErrorInvalidValue;  // the router stays bf16
    case GK_DENSE: return launch_mfma<EPI_STORE, false, true, false, uint16_t>(a, m_tiles, s);
    case GK_DENSE_SITU:
      return launch_mfma<EPI_SITU, true, true, false, uint16_t>(a, m_tiles, s);
    case GK_EXPERT_SITU:
      return launch_mfma<EPI_SITU, true, true, true, uint16_t>(a, m_tiles, s);
    case GK_EXPERT_DOWN:
      return launch_mfma<EPI_STORE, false, true, false, uint16_t>(a, m_tiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
