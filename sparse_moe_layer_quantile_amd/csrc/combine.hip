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
// ascending (the rows of o already carry their routing weight), staged in LDS
// as fp32, then n = y_lat / sqrt(mean(y_lat^2) + eps) * gamma.
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool BF16>
__global__ void __launch_bounds__(256) combine_norm_kernel(const void *__restrict__ o_,
                                                           const int32_t *__restrict__ inv_perm,
                                                           int64_t bt, int k, int L,
                                                           const float *__restrict__ gamma,
                                                           float eps, void *__restrict__ n_) {
  extern __shared__ float ys_all[];  // [4][L]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= bt) return;
  float *ys = ys_all + wave * L;
  constexpr int V = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int nch = L / V;
  const int32_t *ip = inv_perm + t * k;
  float ss = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t pos = ip[j];
      if constexpr (BF16) {
        const uint4 v = reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(o_) + pos * L)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += bf16_to_f32((uint16_t)(w[q] & 0xFFFFu));
          acc[2 * q + 1] += bf16_to_f32((uint16_t)(w[q] >> 16));
        }
      } else {
        const float4 v =
            reinterpret_cast<const float4 *>(static_cast<const float *>(o_) + pos * L)[c];
        acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
      }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      ys[c * V + i] = acc[i];
      ss += acc[i] * acc[i];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = 1.0f / sqrtf(ss / (float)L + eps);
  for (int c = lane; c < nch; c += 64) {
    if constexpr (BF16) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int l = c * V + 2 * q;
        w[q] = pack_bf16x2(ys[l] * inv * gamma[l], ys[l + 1] * inv * gamma[l + 1]);
      }
      reinterpret_cast<uint4 *>(static_cast<uint16_t *>(n_) + t * L)[c] =
          make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float4 v;
      const int l = c * V;
      v.x = ys[l] * inv * gamma[l];
      v.y = ys[l + 1] * inv * gamma[l + 1];
      v.z = ys[l + 2] * inv * gamma[l + 2];
      v.w = ys[l + 3] * inv * gamma[l + 3];
      reinterpret_cast<float4 *>(static_cast<float *>(n_) + t * L)[c] = v;
    }
  }
}

hipError_t launch_combine_norm(const void *o, bool bf16, const int32_t *inv_perm, int64_t bt,
                               int64_t k, int64_t L, const float *gamma, float eps, void *n,
                               hipStream_t s) {
  if (bt <= 0) return hipSuccess;
  const dim3 grid((unsigned)((bt + 3) / 4)), block(256);
  const size_t lds = sizeof(float) * 4 * (size_t)L;
  if (bf16)
    return launch_kernel(combine_norm_kernel<true>, grid, block, lds, s, o, inv_perm, bt, (int)k,
                         (int)L, gamma, eps, n);
  return launch_kernel(combine_norm_kernel<false>, grid, block, lds, s, o, inv_perm, bt, (int)k,
                       (int)L, gamma, eps, n);
}

}  // namespace moe
