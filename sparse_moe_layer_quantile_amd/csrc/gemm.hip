// gemm.hip -- instantiation and launch of the GEMM engine (see gemm.h).
#include <cstdlib>

#include "gemm.h"
#include "gemm2.h"
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

static int env_int(const char *name, int dflt) {
  const char *v = std::getenv(name);
  return v ? std::atoi(v) : dflt;
}

// ---- direct-to-LDS bf16 engine ----------------------------------------------------
struct DmaShape {
  int wm, wn, subm, frn, bk, stages, occ;
  constexpr int threads() const { return 64 * wm * wn; }
  constexpr int tm() const { return wm * subm * 32; }
  constexpr int tn() const { return wn * frn * 32; }
  constexpr size_t lds() const { return (size_t)stages * (tm() + tn()) * bk * 2; }
};
constexpr DmaShape kDma[] = {
    {1, 4, 5, 2, 64, 3, 1},  // 0: 160 x 256, BK 64, 3 stages (156 KB)
    {2, 2, 4, 4, 64, 2, 1},  // 1: 256 x 256, BK 64, 2 stages (128 KB)
    {1, 4, 4, 2, 64, 3, 1},  // 2: 128 x 256, BK 64, 3 stages (144 KB)
    {2, 2, 4, 2, 32, 3, 2},  // 3: 256 x 128, BK 32, 3 stages (72 KB), 2 per CU
    {2, 2, 4, 4, 32, 4, 1},  // 4: 256 x 256, BK 32, 4 stages (128 KB)
    {1, 4, 4, 2, 32, 3, 2},  // 5: 128 x 256, BK 32, 3 stages (72 KB), 2 per CU
    {2, 2, 2, 2, 64, 2, 2},  // 6: 128 x 128, BK 64, 2 stages (64 KB), 2 per CU
    {2, 2, 5, 2, 32, 4, 1},  // 7: 320 x 128, BK 32, 4 stages (112 KB)
    {2, 4, 5, 2, 64, 2, 1},  // 8: 320 x 256, 8 waves, BK 64, 2 stages (144 KB)
    {2, 4, 3, 2, 64, 2, 1},  // 9: 192 x 256, 8 waves, BK 64, 2 stages (112 KB)
    {2, 4, 4, 2, 64, 2, 1},  // 10: 256 x 256, 8 waves, BK 64, 2 stages (128 KB)
    {2, 4, 4, 2, 32, 4, 1},  // 11: 256 x 256, 8 waves, BK 32, 4 stages (128 KB)
};
constexpr int kNumDma = sizeof(kDma) / sizeof(kDma[0]);

template <int V, int EPI, bool DUAL, bool GATHER, bool MSEG, typename OutT>
static hipError_t launch_dma_v(GemmArgs a, hipStream_t s) {
  constexpr DmaShape sh = kDma[V];
  auto kern = g2::gemm_dma_kernel<sh.wm, sh.wn, sh.subm, sh.frn, sh.bk, sh.stages, sh.occ, EPI,
                                  DUAL, GATHER, MSEG, OutT>;
  constexpr size_t lds = sh.lds() + g2::epilogue_lds_bytes<EPI, sh.tm()>();
  static_assert(lds <= 160 * 1024, "LDS of a gfx950 workgroup");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tn_out = DUAL ? sh.tn() / 2 : sh.tn();
  a.n_tiles_n = (int32_t)((a.N + tn_out - 1) / tn_out);
  // dense rasterisation groups (grouped problems group by expert)
  a.group_m = env_int("MOE_GROUP_M_DENSE", 4);
  if (a.group_m < 1) a.group_m = 1;
  int64_t m_tiles;
  if (a.offsets == nullptr) m_tiles = (a.M + sh.tm() - 1) / sh.tm();
  else m_tiles = (a.M + sh.tm() - 1) / sh.tm() + a.n_experts;  // upper bound
  int64_t blocks = m_tiles * a.n_tiles_n;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks <= 0) return hipSuccess;
  return launch_kernel(kern, dim3((unsigned)blocks), dim3(sh.threads()), lds, s, a);
}

template <int EPI, bool DUAL, bool GATHER, typename OutT, bool MSEG = false>
static hipError_t launch_dma(int v, const GemmArgs &a, hipStream_t s) {
  switch (v) {
    case 0: return launch_dma_v<0, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 1: return launch_dma_v<1, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 2: return launch_dma_v<2, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 3: return launch_dma_v<3, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 4: return launch_dma_v<4, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 5: return launch_dma_v<5, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 6: return launch_dma_v<6, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 7: return launch_dma_v<7, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 8: return launch_dma_v<8, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 9: return launch_dma_v<9, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 10: return launch_dma_v<10, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 11: return launch_dma_v<11, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
  }
  return hipErrorInvalidValue;
}

// Tile shape of the bf16 engine per kind (a tuning override is read from
// MOE_GEMM_DENSE / MOE_GEMM_GROUPED).
int dma_variant(GemmKind kind) {
  const int dense = env_int("MOE_GEMM_DENSE", 10);
  const int grouped = env_int("MOE_GEMM_GROUPED", 8);
  const int v = (kind == GK_EXPERT_SITU || kind == GK_EXPERT_DOWN) ? grouped : dense;
  return (v >= 0 && v < kNumDma) ? v : 0;
}

int grouped_tile_rows(int path, bool fp8) {
  if (path == PATH_F32) return sf::BM;
  if (fp8) return mf::BM;
  return kDma[dma_variant(GK_EXPERT_SITU)].tm();
}

// The contractions of the layer, by kind.
hipError_t gemm_launch(const GemmArgs &a, int path, GemmKind kind, bool fp8, int64_t m_tiles,
                       hipStream_t s) {
  if (path == PATH_BF16 && !fp8) {
    const int v = dma_variant(kind);
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
  if (!fp8) {
    switch (kind) {
      case GK_ROUTER: return launch_mfma<EPI_ROUTER, false, false, false, float>(a, m_tiles, s);
      case GK_DENSE: return launch_mfma<EPI_STORE, false, false, false, uint16_t>(a, m_tiles, s);
      case GK_DENSE_SITU:
        return launch_mfma<EPI_SITU, true, false, false, uint16_t>(a, m_tiles, s);
      case GK_EXPERT_SITU:
        return launch_mfma<EPI_SITU, true, false, true, uint16_t>(a, m_tiles, s);
      case GK_EXPERT_DOWN:
        return launch_mfma<EPI_STORE, false, false, false, uint16_t>(a, m_tiles, s);
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
        return launch_mfma<EPI_STORE, false, true, false, uint16_t>(a, m_tiles, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
