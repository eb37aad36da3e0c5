// gemm_api.hip -- moe_gemm_bf16: one bf16 contraction on the direct-to-LDS
// engine, with either operand stored K-outer, fp32 output -- the forms the
// backward pass runs its contractions in.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gemm.h"
#include "gemm_launch.h"
#include "kernels.h"
#include "moe.h"

using namespace moe;

MOE_API moe_status moe_gemm_bf16(const moe_gemm_desc *g, void *stream) {
  if (!g || g->M < 0 || g->N < 0 || g->K < 0 || g->n_experts < 0) return MOE_ERR_INVALID_ARG;
  const bool batched = g->k_offsets != nullptr;
  if (g->M == 0 || g->N == 0 || (!batched && g->K == 0)) {
    if (g->M > 0 && g->N > 0 && !g->c_in && !batched) {
      // no K: C = 0 (a fill kernel, so that the call can be captured in a graph)
      if (!g->c) return MOE_ERR_INVALID_ARG;
      return launch_copy_or_zero_f32(g->c, nullptr, g->ldc * g->M, static_cast<hipStream_t>(stream)) ==
                     hipSuccess
                 ? MOE_OK
                 : MOE_ERR_HIP;
    }
    if (!batched) return MOE_OK;
  }
  if (!g->a || !g->b || !g->c) return MOE_ERR_INVALID_ARG;
  const bool ako = g->a_kouter != 0, bko = g->b_kouter != 0;
  if (g->lda < (ako ? g->M : g->K) || g->ldb < (bko ? g->N : g->K) || g->ldc < g->N)
    return MOE_ERR_INVALID_ARG;
  // 16-byte rows chunks: K-outer operands' rows and the K-inner ones' K
  if ((ako ? g->M : g->K) % 8 || (bko ? g->N : g->K) % 8 || g->lda % 8 || g->ldb % 8)
    return MOE_ERR_UNSUPPORTED;
  // K-inner operands read whole 64-wide K tiles (K-outer rows past K are masked)
  if ((!ako || !bko) && g->K % 64) return MOE_ERR_UNSUPPORTED;
  if (batched && (!ako || !bko || g->n_experts == 0)) return MOE_ERR_INVALID_ARG;
  if (ako && !bko) return MOE_ERR_UNSUPPORTED;
  // 32-bit lane offsets within a K tile
  if (64 * std::max(g->lda, g->ldb) * 2 >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  GemmArgs a = {};
  a.M = g->M;
  a.N = g->N;
  a.nseg = 1;
  a.seg[0] = GemmSeg{g->a, g->lda, g->b, g->ldb, nullptr, g->K};
  a.out = g->c;
  a.ldo = g->ldc;
  a.resid = g->c_in;
  a.ldr = g->ldc;
  a.beta = a.beta_u = a.inv_beta = a.inv_beta_u = 1.0f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (batched) {
    if (g->c_in) return MOE_ERR_UNSUPPORTED;
    a.offsets = g->k_offsets;
    a.n_experts = (int32_t)g->n_experts;
    e = launch_dma_ko<EPI_STORE, true, true, true, false, float>(kgrp_variant(), a, s);
  } else if (ako) {
    e = launch_dma_ko<EPI_STORE, true, true, false, false, float>(kVDense, a, s);
  } else if (bko) {
    e = launch_dma_ko<EPI_STORE, false, true, false, false, float>(g->M <= 64 ? kVSmallM : kVDense,
                                                                  a, s);
  } else {
    e = launch_dma<EPI_STORE, false, false, float, false>(g->M <= 64 ? kVSmallM : kVDense, a, s);
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
