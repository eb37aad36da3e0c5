// kernels.h -- internal launch interface between the C ABI (api.hip) and the
// kernels.  Every launcher enqueues on the given stream and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct GemmArgs;

enum GemmPath { PATH_BF16 = 0, PATH_F32 = 1 };
enum GemmKind {
  GK_ROUTER = 0,       // z = A B^T + bias -> fp32 (+ transposed copy)
  GK_DENSE = 1,        // C = A B^T (K may be split over segments)
  GK_DENSE_SITU = 2,   // h = SiTU(A Bg^T, A Bu^T)
  GK_EXPERT_SITU = 3,  // grouped + gathered A, SiTU epilogue
  GK_EXPERT_DOWN = 4,  // grouped, plain store (h rows already carry the routing weight)
};

int gemm_bm(int path);
// Storage format of a GEMM's weights (B operand): bf16 (fp32 on the fp32
// path), fp8 e4m3 with 128 x 128 block scales, MXFP4 with E8M0 scales per 32
// (WF_MX4A8: and the A operand in MX FP8, for the block-scaled MFMA); WF_MX8A8:
// MX FP8 (e4m3 with E8M0 scales per 32) for both operands.
enum WFmt { WF_BF16 = 0, WF_FP8 = 1, WF_MX4 = 2, WF_MX4A8 = 3, WF_MX8A8 = 4 };
// M-tile rows of the grouped GEMMs for rows (token, expert) pairs over
// n_experts experts with weights in format wf (the dispatch lays its tile
// table out in these units).
int grouped_tile_rows(int path, int wf, int64_t rows, int64_t n_experts);
// Tile shape (index into the direct-to-LDS engine's shape table) of a bf16
// problem of this kind over `rows` rows (per expert: n_experts).
int dma_variant(GemmKind kind, int64_t rows, int64_t n_experts);
int gemm_bn_out(int path, bool dual);
hipError_t gemm_launch(const GemmArgs &a, int path, GemmKind kind, int wf, int64_t m_tiles,
                       hipStream_t s);

// ---- routing ------------------------------------------------------------------
// zT [E][bt] fp32 -> alpha[e] = m-th largest of row e.
hipError_t launch_quantile(const float *zT, int64_t bt, int64_t n_experts, int64_t m,
                           float *alpha, hipStream_t s);
// z [bt][E] fp32, alpha [E] or NULL -> idx [bt][k] ascending, w [bt][k] = sigmoid(z).
hipError_t launch_topk(const float *z, const float *alpha, int64_t bt, int64_t n_experts,
                       int64_t k, int32_t *idx, float *w, hipStream_t s);
// dst[i] = src ? src[i] : 0 for i < n.
hipError_t launch_copy_or_zero_f32(float *dst, const float *src, int64_t n, hipStream_t s);
// alpha[i] += rate * (zeta[i] - alpha[i]) in fp32, each operation rounded
hipError_t launch_cutoff_update(float *alpha, const float *zeta, int64_t n, float rate,
                                hipStream_t s);
hipError_t launch_zero_i32(int32_t *dst, int64_t n, hipStream_t s);

// ---- dispatch -------------------------------------------------------------------
// masks: [E][ceil(bt/64)] u64 scratch; counts must be zeroed first.
// w / w_sorted may be NULL; otherwise w_sorted[pos] = w[perm[pos]].
hipError_t launch_dispatch(const int32_t *idx, const float *w, int64_t bt, int64_t k,
                           int64_t n_experts, int tile_bm, uint64_t *masks, int32_t *counts,
                           int32_t *offsets, int32_t *tile_offsets, int32_t *perm,
                           int32_t *inv_perm, float *w_sorted, hipStream_t s);

// ---- MX FP8 activations -------------------------------------------------------------
// x: n bf16 elements (n a multiple of 32, 16-byte aligned) -> codes[n] E4M3 and
// scales[n / 32] E8M0 (OCP MX, blocks of 32 consecutive elements).
hipError_t launch_mx8_quant(const void *x, int64_t n, uint8_t *codes, uint8_t *scales,
                            hipStream_t s);

// ---- combine + latent RMSNorm ---------------------------------------------------
// o [P][L] (act) rows already scaled by their routing weight; n [bt][L] (act).
hipError_t launch_combine_norm(const void *o, bool bf16, const int32_t *inv_perm, int64_t bt,
                               int64_t k, int64_t L, const float *gamma, float eps, void *n,
                               hipStream_t s);

}  // namespace moe
