// gemm_launch.h -- tile shapes of the direct-to-LDS engine and its host-side
// launch templates (instantiated in the gemm_dma_*.hip units, dispatched from
// gemm.hip).
#pragma once

#include <algorithm>
#include <cstdlib>

#include "gemm.h"
#include "gemm2.h"
#include "kernels.h"

namespace moe {

inline int env_int(const char *name, int dflt) {
  const char *v = std::getenv(name);
  return v ? std::atoi(v) : dflt;
}

// ---- direct-to-LDS bf16 engine ----------------------------------------------------
struct DmaShape {
  int wm, wn, subm, frn, bk, stages, occ;  // occ: minimum waves per SIMD (launch bound)
  int ma = 0;  // rows of a short tile (0: wm * subm * 32)
  constexpr int threads() const { return 64 * wm * wn; }
  constexpr int tm() const { return ma > 0 ? ma : wm * subm * 32; }
  constexpr int tn() const { return wn * frn * 32; }
  // bytes of a B tile row in format bf (g2::BFmt): bf16, fp8 codes, MXFP4 bytes
  static constexpr int b_row_bytes(int bk, int bf) {
    return (bf == g2::BF_FP8 || bf == g2::BF_MX8A8)    ? bk
           : (bf == g2::BF_MX4 || bf == g2::BF_MX4A8) ? bk / 2
                                                      : bk * 2;
  }
  // scale-code instructions (256 bytes) of `rows` rows of bk/32 codes, in whole
  // rounds of the workgroup's waves
  constexpr size_t code_bytes(int rows) const {
    const int nw = wm * wn;
    return (size_t)((rows * (bk / 32) + 255) / 256 + nw - 1) / nw * nw * 256;
  }
  // stage ring: A rows (bf16, or e4m3 codes with MX FP8 A) and B rows; MXFP4 B
  // with K tiles of 128 or more also the B rows' E8M0 codes, MX FP8 A the A rows'
  constexpr size_t lds(int bf = g2::BF_BF16) const {
    const bool a8 = bf == g2::BF_MX4A8 || bf == g2::BF_MX8A8;
    const bool mx = bf == g2::BF_MX4 || a8;
    return (size_t)stages * (tm() * bk * (a8 ? 1 : 2) + tn() * b_row_bytes(bk, bf) +
                             (mx && bk >= 128 ? code_bytes(tn()) : 0) +
                             (a8 ? code_bytes(tm()) : 0));
  }
  // every wave issues whole rounds of A and of B DMA instructions (1 KB each)
  constexpr bool whole_rounds(int bf = g2::BF_BF16) const {
    return (tm() / (512 / bk)) % (wm * wn) == 0 &&
           (tn() / (1024 / b_row_bytes(bk, bf))) % (wm * wn) == 0;
  }
};
constexpr DmaShape kDma[] = {
    {2, 4, 5, 2, 64, 2, 1},  // 0: 320 x 256, 8 waves, BK 64, 2 stages (144 KB)
    {2, 4, 3, 2, 64, 2, 1},  // 1: 192 x 256, 8 waves, BK 64, 2 stages (112 KB)
    {2, 4, 4, 2, 64, 2, 1},  // 2: 256 x 256, 8 waves, BK 64, 2 stages (128 KB)
    {1, 4, 1, 2, 64, 4, 1},  // 3: 32 x 256, 4 waves, BK 64, 4 stages (144 KB)
    // measured alternatives (slower on the K3 shapes), kept for tuning
    {2, 4, 5, 2, 32, 4, 1},  // 4: 320 x 256, 8 waves, BK 32, 4 stages (144 KB)
    {1, 4, 5, 2, 64, 3, 1},  // 5: 160 x 256, 4 waves, BK 64, 3 stages (156 KB)
    // MXFP4 B (a quarter of the bf16 B bytes a stage): a deeper ring keeps as
    // many weight bytes in flight when a few rows stream the weights
    {1, 4, 1, 2, 64, 8, 1},  // 6: 32 x 256, 4 waves, BK 64, 8 stages (96 KB + 32 KB scales)
    // 7: 8 x 256 short tile (decode), BK 128: 64 bytes of each weight row and
    //    its 4 scale codes a stage, 8 stages (152 KB)
    {1, 4, 1, 2, 128, 8, 1, 8},
    // 8: the same with BK 256: a whole 128-byte line of each weight row and its
    //    8 scale codes a stage, 4 stages (152 KB); for K a multiple of 256
    {1, 4, 1, 2, 256, 4, 1, 8},
    // quantised B (fp8, MXFP4): B stages a half or a quarter of bf16's leave
    // room for a third stage of the grouped tiles
    {2, 4, 4, 2, 64, 3, 1},  // 9: 256 x 256, BK 64, 3 stages
    {2, 4, 3, 2, 64, 3, 1},  // 10: 192 x 256, BK 64, 3 stages
    // MX FP8 A x MXFP4 B (block-scaled MFMA): K tiles of 128 (two 64-wide MFMA
    // k steps), both operands' E8M0 codes in the stage
    {2, 4, 4, 2, 128, 3, 1},  // 11: 256 x 256, 3 stages (156 KB)
    {2, 4, 5, 2, 128, 2, 1},  // 12: 320 x 256, 2 stages (120 KB)
    {2, 4, 3, 2, 128, 3, 1},  // 13: 192 x 256, 3 stages (132 KB)
    // MX FP8 A x MX FP8 B (twice the B bytes of MXFP4): 2-stage rings
    {2, 4, 4, 2, 128, 2, 1},  // 14: 256 x 256 (136 KB)
    {2, 4, 3, 2, 128, 2, 1},  // 15: 192 x 256 (120 KB)
    // expert-batched weight gradients (few K tiles, then a large fp32 store):
    // a small ring and at most 128 VGPRs, so that two workgroups share a CU
    // and one's stores drain while the other loads and multiplies.  Against
    // the 256 x 256 shape, 2-stage rings and 128 x 128 tiles with two or four
    // workgroups a CU: the backward 2-3% faster at K3 prefill, 8-10% at decode
    {2, 4, 2, 2, 32, 3, 4},  // 16: 128 x 256, 8 waves, BK 32, 3 stages (72 KB)
    // fp8 B, grouped: one wave row of 8 waves along N, so each B element is
    // widened by one wave only, with 5 x 2 MFMA blocks a wave (K3 fp8 prefill
    // expert gate/up 6.90 ms against 7.50 ms on 192 x 256, 3 stages; 7.05 ms
    // with 2 stages)
    {1, 8, 5, 2, 64, 3, 1},  // 17: 160 x 512, BK 64, 3 stages (156 KB)
};
// the shapes the engine picks by default (gemm.hip, dma_variant)
constexpr int kVGrouped = 0, kVGroupedShort = 1, kVDense = 2, kVSmallM = 3, kVSmallMX4 = 6,
              kVTinyMX4 = 7, kVTinyMX4W = 8, kVQ256 = 9, kVQ192 = 10, kVA8 = 11,
              kVA8W = 12, kVA8S = 13, kVB8 = 14, kVB8S = 15, kVKgrp = 16, kVF8W = 17;
constexpr int kNumDma = sizeof(kDma) / sizeof(kDma[0]);
// the shape of the expert-batched weight gradients (MOE_KGRP_V overrides it)
inline int kgrp_variant() { return env_int("MOE_KGRP_V", kVKgrp); }
// shapes a bf16 B operand can take (6..8 are MXFP4-only)
constexpr bool bf16_shape(int v) { return v >= 0 && v < 6; }

template <int V, int EPI, bool DUAL, bool GATHER, bool MSEG, int BF, typename OutT,
          bool AKO = false, bool BKO = false, bool KGRP = false>
hipError_t launch_dma_impl(GemmArgs a, hipStream_t s) {
  constexpr DmaShape sh = kDma[V];
  auto kern = g2::gemm_dma_kernel<sh.wm, sh.wn, sh.subm, sh.frn, sh.bk, sh.stages, sh.occ, sh.ma,
                                  EPI, DUAL, GATHER, MSEG, BF, OutT, AKO, BKO, KGRP>;
  constexpr size_t lds = sh.lds(BF) + g2::extra_lds_bytes<EPI, sh.tm(), sh.tn(), BF, sh.bk>();
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
  // short tiles of a grouped problem run nper consecutive N tiles in one
  // workgroup (the kernel's persistent-N form: bf16 or MXFP4 B with in-stage
  // scales), nper dividing the N tiles of whole tiles only
  a.nper = 1;
  if constexpr (sh.ma > 0 && BF != g2::BF_FP8 && EPI != EPI_ROUTER &&
                (BF != g2::BF_MX4 || sh.bk >= 128)) {
    if (a.offsets != nullptr && a.N % tn_out == 0) {
      // two workgroups a (expert, M tile): half the N tiles each, or the
      // largest divisor below (K3 MXFP4 decode, gate/up 24 tiles / down 14:
      // 1.30 / 0.69 ms against 1.36 / 0.68 ms with up to 8 and 1.42 / 0.76 ms
      // with all of them in one workgroup)
      int nper = env_int("MOE_GEMM_NPER", 0);
      if (nper <= 0) nper = std::max(1, (int)(a.n_tiles_n / 2));
      while (nper > 1 && a.n_tiles_n % nper) --nper;
      a.nper = nper;
      a.n_tiles_n /= nper;
    }
  }
  // dense rasterisation groups (grouped problems group by expert)
  a.group_m = env_int("MOE_GROUP_M_DENSE", 4);
  if (a.group_m < 1) a.group_m = 1;
  int64_t m_tiles;
  if (KGRP) m_tiles = (a.M + sh.tm() - 1) / sh.tm() * a.n_experts;  // every expert's [M][N]
  else if (a.offsets == nullptr) m_tiles = (a.M + sh.tm() - 1) / sh.tm();
  else m_tiles = (a.M + sh.tm() - 1) / sh.tm() + a.n_experts;  // upper bound
  int64_t blocks = m_tiles * a.n_tiles_n;
  // split K when a dense problem has too few tiles to spread its weight
  // stream over the chip (short batches): about 256 workgroups, two or more
  // K tiles each, within the partial-sum buffer
  a.ksplit = 1;
  if (!KGRP && a.offsets == nullptr && a.partial != nullptr && blocks > 0 && blocks < 128) {
    int64_t ktiles = 0;
    for (int i = 0; i < a.nseg; ++i) ktiles += (a.seg[i].k + sh.bk - 1) / sh.bk;
    const int64_t ldp = DUAL ? 2 * a.N : a.N;
    int64_t ks = std::min((256 + blocks - 1) / blocks, ktiles / 2);
    ks = std::min(ks, a.partial_cap / (a.M * ldp));
    if (ks > 1) {
      const int64_t kper = (ktiles + ks - 1) / ks;
      a.ksplit = (int32_t)((ktiles + kper - 1) / kper);  // every split gets K tiles
      a.ldp = ldp;
    }
  }
  blocks = (blocks + 7) / 8 * 8;
  if (blocks <= 0) return hipSuccess;
  hipError_t e = launch_kernel(kern, dim3((unsigned)blocks, (unsigned)a.ksplit),
                               dim3(sh.threads()), lds, s, a);
  if (e != hipSuccess || a.ksplit <= 1) return e;
  const unsigned rblocks = (unsigned)std::min<int64_t>((a.M * a.N + 255) / 256, 8192);
  return launch_kernel(g2::splitk_reduce_kernel<EPI, DUAL, OutT>, dim3(rblocks), dim3(256), 0, s,
                       a);
}

template <int V, int EPI, bool DUAL, bool GATHER, bool MSEG, typename OutT>
hipError_t launch_dma_v(const GemmArgs &a, hipStream_t s) {
  // K-segmented problems need whole DMA rounds per wave: else the 256 x 256 shape
  if constexpr (MSEG && !kDma[V].whole_rounds())
    return launch_dma_impl<kVDense, EPI, DUAL, GATHER, MSEG, g2::BF_BF16, OutT>(a, s);
  else
    return launch_dma_impl<V, EPI, DUAL, GATHER, MSEG, g2::BF_BF16, OutT>(a, s);
}

// fp8 e4m3 B with block scales: the shape for the variant v the bf16 engine
// would take (for the short grouped tiles, 160 x 512 with a third stage, which
// the half-size B stage leaves room for; the other grouped and small-M ones as
// they are, the dense one otherwise); MOE_GEMM_FP8 overrides the grouped shape
inline int fp8_shape(int v, bool grouped) {
  const int dflt = v == kVGroupedShort                          ? kVF8W
                   : (v == kVGrouped || v == kVSmallM) ? v
                                                                : kVDense;
  const int o = grouped ? env_int("MOE_GEMM_FP8", -1) : -1;
  return (o == kVGrouped || o == kVGroupedShort || o == kVSmallM || o == kVQ256 || o == kVQ192 ||
          o == kVF8W)
             ? o
             : dflt;
}
template <int EPI, bool DUAL, bool GATHER, typename OutT, bool MSEG = false>
hipError_t launch_dma_b8(int shape, const GemmArgs &a, hipStream_t s) {
  constexpr int F = g2::BF_FP8;
  static_assert(!MSEG || kDma[kVDense].whole_rounds(F), "segmented fp8 shape");
  if constexpr (MSEG) return launch_dma_impl<kVDense, EPI, DUAL, GATHER, true, F, OutT>(a, s);
  switch (shape) {
    case kVGrouped: return launch_dma_impl<kVGrouped, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVGroupedShort:
      return launch_dma_impl<kVGroupedShort, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVSmallM: return launch_dma_impl<kVSmallM, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVQ256: return launch_dma_impl<kVQ256, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVQ192: return launch_dma_impl<kVQ192, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVF8W: return launch_dma_impl<kVF8W, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    default: return launch_dma_impl<kVDense, EPI, DUAL, GATHER, false, F, OutT>(a, s);
  }
}

// MXFP4 B (routed experts): the shape for the variant v the bf16 engine would
// take for `rows` pairs over n_experts: the grouped shapes as they are; for
// few rows a deeper-ring 32-row shape, and the 8-row short tile when experts
// hold about two rows each (decode); MOE_GEMM_MX4 overrides
inline int mx4_shape(int v, int64_t rows, int64_t n_experts) {
  const int dflt = v == kVGrouped        ? kVGrouped
                   : v != kVSmallM       ? kVGroupedShort
                   : rows <= 2 * n_experts ? kVTinyMX4
                                           : kVSmallMX4;
  const int o = env_int("MOE_GEMM_MX4", -1);
  return (o == kVGrouped || o == kVGroupedShort || o == kVSmallMX4 || o == kVTinyMX4 ||
          o == kVQ256 || o == kVQ192)
             ? o
             : dflt;
}
// (the 8-row short tile takes its 256-wide K tiles where K allows; both forms
// have 8-row tiles, so the dispatch's tile table is the same)
template <int EPI, bool DUAL, bool GATHER, typename OutT>
hipError_t launch_dma_b4(int shape, const GemmArgs &a, hipStream_t s) {
  constexpr int F = g2::BF_MX4;
  if (shape == kVTinyMX4 && a.seg[0].k % 256 == 0 && env_int("MOE_GEMM_MX4_BK128", 0) == 0)
    shape = kVTinyMX4W;
  switch (shape) {
    case kVGrouped: return launch_dma_impl<kVGrouped, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVSmallMX4: return launch_dma_impl<kVSmallMX4, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVTinyMX4: return launch_dma_impl<kVTinyMX4, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVTinyMX4W: return launch_dma_impl<kVTinyMX4W, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVQ256: return launch_dma_impl<kVQ256, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVQ192: return launch_dma_impl<kVQ192, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    default: return launch_dma_impl<kVGroupedShort, EPI, DUAL, GATHER, false, F, OutT>(a, s);
  }
}

template <int EPI, bool DUAL, bool GATHER, typename OutT, bool MSEG = false>
hipError_t launch_dma(int v, const GemmArgs &a, hipStream_t s) {
  switch (v) {
    case 0: return launch_dma_v<0, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 1: return launch_dma_v<1, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 2: return launch_dma_v<2, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 3: return launch_dma_v<3, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 4: return launch_dma_v<4, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
    case 5: return launch_dma_v<5, EPI, DUAL, GATHER, MSEG, OutT>(a, s);
  }
  return hipErrorInvalidValue;
}

// Operands stored K-outer (the backward pass): AKO: A is [K][M], BKO: B is
// [K][N] (per expert for a grouped problem), both bf16; KGRP: the routed
// experts' weight gradients, one [M][N] output per expert over its pair rows
// (offsets) of K-outer A and B.  fp32 output.  K-outer A takes the dense
// shape (and the weight gradients' own); K-outer B every bf16 shape.
template <int EPI, bool AKO, bool BKO, bool KGRP, bool GATHER, typename OutT>
hipError_t launch_dma_ko(int v, const GemmArgs &a, hipStream_t s) {
  constexpr int F = g2::BF_BF16;
  if constexpr (AKO) {
    if constexpr (KGRP) {
      if (v == kVKgrp)
        return launch_dma_impl<kVKgrp, EPI, false, GATHER, false, F, OutT, AKO, BKO, KGRP>(a, s);
    }
    return launch_dma_impl<kVDense, EPI, false, GATHER, false, F, OutT, AKO, BKO, KGRP>(a, s);
  } else {
    switch (v) {
      case kVGrouped:
        return launch_dma_impl<kVGrouped, EPI, false, GATHER, false, F, OutT, AKO, BKO, KGRP>(a, s);
      case kVGroupedShort:
        return launch_dma_impl<kVGroupedShort, EPI, false, GATHER, false, F, OutT, AKO, BKO, KGRP>(
            a, s);
      case kVSmallM:
        return launch_dma_impl<kVSmallM, EPI, false, GATHER, false, F, OutT, AKO, BKO, KGRP>(a, s);
      default:
        return launch_dma_impl<kVDense, EPI, false, GATHER, false, F, OutT, AKO, BKO, KGRP>(a, s);
    }
  }
}
#define MOE_KO_KINDS(X)                         \
  X(EPI_STORE, false, true, false, false, float) \
  X(EPI_STORE, false, true, false, true, float)  \
  X(EPI_STORE, true, true, false, false, float)  \
  X(EPI_STORE, true, true, true, false, float)
#define MOE_KO_EXTERN(E, A, B, K, G, T) \
  extern template hipError_t launch_dma_ko<E, A, B, K, G, T>(int, const GemmArgs &, hipStream_t);
MOE_KO_KINDS(MOE_KO_EXTERN)

// launch_dma instantiations, one per problem kind (gemm_dma_*.hip)
#define MOE_DMA_KINDS(X)                                  \
  X(EPI_ROUTER, false, false, float, false)               \
  X(EPI_STORE, false, false, uint16_t, true)              \
  X(EPI_STORE, false, false, uint16_t, false)             \
  X(EPI_SITU, true, false, uint16_t, false)               \
  X(EPI_SITU, true, true, uint16_t, false)                \
  X(EPI_STORE, false, false, float, false)                \
  X(EPI_STORE, false, true, float, false)
#define MOE_DMA_EXTERN(E, D, G, T, M) \
  extern template hipError_t launch_dma<E, D, G, T, M>(int, const GemmArgs &, hipStream_t);
MOE_DMA_KINDS(MOE_DMA_EXTERN)
#define MOE_B8_KINDS(X)                      \
  X(EPI_STORE, false, false, uint16_t, false) \
  X(EPI_STORE, false, false, uint16_t, true)  \
  X(EPI_SITU, true, false, uint16_t, false)   \
  X(EPI_SITU, true, true, uint16_t, false)
#define MOE_B8_EXTERN(E, D, G, T, M) \
  extern template hipError_t launch_dma_b8<E, D, G, T, M>(int, const GemmArgs &, hipStream_t);
MOE_B8_KINDS(MOE_B8_EXTERN)
// MX FP8 A x MXFP4 B, the routed experts on the block-scaled MFMA: the tile
// rows by the rows an expert holds on average (override MOE_GEMM_A8: 11-13)
inline int a8_shape(int64_t rows, int64_t n_experts) {
  const int dflt = rows <= 200 * n_experts ? kVA8S : rows <= 300 * n_experts ? kVA8W : kVA8;
  const int v = env_int("MOE_GEMM_A8", dflt);
  return (v == kVA8 || v == kVA8W || v == kVA8S) ? v : dflt;
}
template <int EPI, bool DUAL, bool GATHER, typename OutT>
hipError_t launch_dma_b4a8(int shape, const GemmArgs &a, hipStream_t s) {
  constexpr int F = g2::BF_MX4A8;
  switch (shape) {
    case kVA8W: return launch_dma_impl<kVA8W, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVA8S: return launch_dma_impl<kVA8S, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    default: return launch_dma_impl<kVA8, EPI, DUAL, GATHER, false, F, OutT>(a, s);
  }
}
extern template hipError_t launch_dma_b4a8<EPI_STORE, false, false, uint16_t>(int,
                                                                            const GemmArgs &,
                                                                            hipStream_t);
extern template hipError_t launch_dma_b4a8<EPI_SITU, true, true, uint16_t>(int, const GemmArgs &,
                                                                         hipStream_t);
// MX FP8 A x MX FP8 B: 320-row tiles for 201-300 rows an expert, else 192
// (<= 200) or 256 (override MOE_GEMM_A8: 12, 14, 15)
inline int mx8_shape(int64_t rows, int64_t n_experts) {
  const int dflt = rows <= 200 * n_experts ? kVB8S : rows <= 300 * n_experts ? kVA8W : kVB8;
  const int v = env_int("MOE_GEMM_A8", dflt);
  return (v == kVA8W || v == kVB8 || v == kVB8S) ? v : dflt;
}
template <int EPI, bool DUAL, bool GATHER, typename OutT>
hipError_t launch_dma_b8a8(int shape, const GemmArgs &a, hipStream_t s) {
  constexpr int F = g2::BF_MX8A8;
  switch (shape) {
    case kVA8W: return launch_dma_impl<kVA8W, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    case kVB8S: return launch_dma_impl<kVB8S, EPI, DUAL, GATHER, false, F, OutT>(a, s);
    default: return launch_dma_impl<kVB8, EPI, DUAL, GATHER, false, F, OutT>(a, s);
  }
}
extern template hipError_t launch_dma_b8a8<EPI_STORE, false, false, uint16_t>(int,
                                                                            const GemmArgs &,
                                                                            hipStream_t);
extern template hipError_t launch_dma_b8a8<EPI_SITU, true, true, uint16_t>(int, const GemmArgs &,
                                                                         hipStream_t);
#define MOE_B4_KINDS(X)                     \
  X(EPI_STORE, false, false, uint16_t)      \
  X(EPI_SITU, true, true, uint16_t)
#define MOE_B4_EXTERN(E, D, G, T) \
  extern template hipError_t launch_dma_b4<E, D, G, T>(int, const GemmArgs &, hipStream_t);
MOE_B4_KINDS(MOE_B4_EXTERN)

}  // namespace moe
