// combine.hip -- score-weighted combine of the routed expert outputs and the
// latent RMSNorm that precedes the up projection.
//
// tech.news18a.com "KimiK3的StableLatentMoE架构解析": figure 2 (latent_norm after
// the experts, before the fusion with the shared path) and the second
// technique, RMSNorm Before Up (the tensor entering up_proj is normalised in
// the latent space); mkdocs.reaper.mx "Vue d'ensemble de l'architecture",
// per-token step f ("RMSNorm + W↑").
//
// One wavefront per token: y_lat = sum_j o[inv_perm[t*k + j]] with j
// ascending (the rows of o already carry their routing weight), held in
// registers as fp32 (NCH 16-byte chunks per lane), then
// n = y_lat / sqrt(mean(y_lat^2) + eps) * gamma.  The k rows of a token are
// read eight at a time, so each lane has up to 8 NCH loads in flight; the
// pass is bound by reading o once.  With inv_perm NULL and k = 1 it is a plain
// RMSNorm of row t (the dense FFN's pre-norm; mkdocs.reaper.mx "Vue d'ensemble
// de l'architecture", section "Ce que fait une couche").
#include "common.h"
#include "kernels.h"

namespace moe {

// GATHER: rows o[inv_perm[t k + j]] (the combine); else row t (plain RMSNorm)
template <bool BF16, int NCH, bool GATHER>
__global__ void __launch_bounds__(256) combine_norm_kernel(const void *__restrict__ o_,
                                                           const int32_t *__restrict__ inv_perm,
                                                           int64_t bt, int k, int L,
                                                           const float *__restrict__ gamma,
                                                           float eps, void *__restrict__ n_) {
  constexpr int V = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= bt) return;
  const int nch = L / V;
  const int32_t *ip = GATHER ? inv_perm + t * k : nullptr;
  float acc[NCH][V];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[c][i] = 0.0f;

  for (int j0 = 0; j0 < k; j0 += 8) {
    int64_t pos[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      pos[u] = j0 + u < k ? (GATHER ? (int64_t)ip[j0 + u] : t) : -1;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = lane + 64 * c;
      if (ch >= nch) continue;
      if constexpr (BF16) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (pos[u] >= 0)
            v[u] = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(o_) +
                                                    pos[u] * L)[ch];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (pos[u] < 0) continue;
          const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[c][2 * q] += bf16_to_f32((uint16_t)(w[q] & 0xFFFFu));
            acc[c][2 * q + 1] += bf16_to_f32((uint16_t)(w[q] >> 16));
          }
        }
      } else {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (pos[u] >= 0)
            v[u] = reinterpret_cast<const float4 *>(static_cast<const float *>(o_) + pos[u] * L)[ch];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (pos[u] < 0) continue;
          acc[c][0] += v[u].x;
          acc[c][1] += v[u].y;
          acc[c][2] += v[u].z;
          acc[c][3] += v[u].w;
        }
      }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < V; ++i) ss += acc[c][i] * acc[c][i];  // unused chunks hold 0
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = 1.0f / sqrtf(ss / (float)L + eps);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch >= nch) continue;
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma) + ch * (V / 4);
    if constexpr (BF16) {
      const float4 ga = g4[0], gb = g4[1];
      const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack_bf16x2(acc[c][2 * q] * inv * g[2 * q], acc[c][2 * q + 1] * inv * g[2 * q + 1]);
      reinterpret_cast<uint4 *>(static_cast<uint16_t *>(n_) + t * L)[ch] =
          make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      const float4 g = g4[0];
      reinterpret_cast<float4 *>(static_cast<float *>(n_) + t * L)[ch] =
          make_float4(acc[c][0] * inv * g.x, acc[c][1] * inv * g.y, acc[c][2] * inv * g.z,
                      acc[c][3] * inv * g.w);
    }
  }
}

template <bool BF16>
static hipError_t launch_cn(const void *o, const int32_t *inv_perm, int64_t bt, int64_t k,
                            int64_t L, const float *gamma, float eps, void *n, hipStream_t s) {
  constexpr int V = BF16 ? 8 : 4;
  const int64_t per_lane = (L / V + 63) / 64;
  const dim3 grid((unsigned)((bt + 3) / 4)), block(256);
  if (inv_perm == nullptr) {  // plain RMSNorm rows (k = 1), up to 16 chunks a lane
    if (per_lane <= 8)
      return launch_kernel(combine_norm_kernel<BF16, 8, false>, grid, block, 0, s, o, inv_perm, bt,
                           (int)k, (int)L, gamma, eps, n);
    if (per_lane <= 16)
      return launch_kernel(combine_norm_kernel<BF16, 16, false>, grid, block, 0, s, o, inv_perm,
                           bt, (int)k, (int)L, gamma, eps, n);
    return hipErrorInvalidValue;
  }
  if (per_lane <= 1)
    return launch_kernel(combine_norm_kernel<BF16, 1, true>, grid, block, 0, s, o, inv_perm, bt,
                         (int)k, (int)L, gamma, eps, n);
  if (per_lane <= 2)
    return launch_kernel(combine_norm_kernel<BF16, 2, true>, grid, block, 0, s, o, inv_perm, bt,
                         (int)k, (int)L, gamma, eps, n);
  if (per_lane <= 4)
    return launch_kernel(combine_norm_kernel<BF16, 4, true>, grid, block, 0, s, o, inv_perm, bt,
                         (int)k, (int)L, gamma, eps, n);
  if (per_lane <= 8)
    return launch_kernel(combine_norm_kernel<BF16, 8, true>, grid, block, 0, s, o, inv_perm, bt,
                         (int)k, (int)L, gamma, eps, n);
  return hipErrorInvalidValue;
}

hipError_t launch_combine_norm(const void *o, bool bf16, const int32_t *inv_perm, int64_t bt,
                               int64_t k, int64_t L, const float *gamma, float eps, void *n,
                               hipStream_t s) {
  if (bt <= 0) return hipSuccess;
  // rows are read as 16-byte chunks: L a multiple of 8 (bf16) or 4 (fp32), at most
  // 8 chunks per lane (16 for a plain RMSNorm: inv_perm NULL, k = 1)
  if (bf16) return launch_cn<true>(o, inv_perm, bt, k, L, gamma, eps, n, s);
  return launch_cn<false>(o, inv_perm, bt, k, L, gamma, eps, n, s);
}

}  // namespace moe
