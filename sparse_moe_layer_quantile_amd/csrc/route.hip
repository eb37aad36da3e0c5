// route.hip -- Quantile Balancing cutoffs and top-k selection.
//
// The router of the Stable LatentMoE (tech.news18a.com
// "KimiK3的StableLatentMoE架构解析", figure 2 and the third technique,
// Quantile Balancing) scores each token against every expert with a sigmoid
// gate, shifts the experts by per-expert cutoffs chosen so that each expert
// receives its quantile share of tokens, and keeps the top 16 of 896
// (mkdocs.reaper.mx "Vue d'ensemble de l'architecture", per-token step c).
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// ---- batch quantile: radix select of the m-th largest value -----------------
// One workgroup per expert.  Four passes over 8-bit digits of the order
// keys, most significant first; each pass histograms the keys that share the
// digits chosen so far and picks the digit holding the m-th largest.
__global__ void __launch_bounds__(256) quantile_kernel(const float *__restrict__ zT, int64_t bt,
                                                       int64_t m, float *__restrict__ alpha) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_digit, sel_rank;
  const int tid = threadIdx.x, lane = tid & 63;
  const float *col = zT + (int64_t)blockIdx.x * bt;
  uint32_t prefix = 0, mask = 0, rank = (uint32_t)m;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int64_t t = tid; t < bt; t += 256) {
      const uint32_t key = f32_order_key(col[t]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns digits 255-4*lane .. 252-4*lane, scanned from the top
      uint32_t c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - 4 * lane - q];
      const uint32_t local = c[0] + c[1] + c[2] + c[3];
      const uint32_t incl = wave_incl_scan_u32(local, lane);
      uint32_t cum = incl - local;
      if (cum < rank && rank <= incl) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + c[q] >= rank) {
            sel_digit = 255u - 4u * lane - q;
            sel_rank = rank - cum;
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= 255u << shift;
    rank = sel_rank;
    __syncthreads();
  }
  if (tid == 0) alpha[blockIdx.x] = order_key_f32(prefix);
}

hipError_t launch_quantile(const float *zT, int64_t bt, int64_t n_experts, int64_t m,
                           float *alpha, hipStream_t s) {
  if (n_experts <= 0 || bt <= 0) return hipSuccess;
  return launch_kernel(quantile_kernel, dim3((unsigned)n_experts), dim3(256), 0, s, zT, bt, m,
                       alpha);
}

// ---- top-k: one wavefront per token -------------------------------------------
// Lane l holds experts l, l+64, ...  Each candidate is the 64-bit key
// (order key of z - alpha) << 32 | ~e, so a maximum picks the largest
// cutoff-adjusted logit and, among equal ones, the lowest expert id.  k rounds
// of a wave maximum take the winners; a ballot prefix then lists them in
// ascending expert id.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

template <int NPL>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ z,
                                                   const float *__restrict__ alpha, int64_t bt,
                                                   int E, int k, int32_t *__restrict__ idx,
                                                   float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= bt) return;
  const float *zr = z + t * E;
  uint64_t cand[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float r = zr[e] - (alpha ? alpha[e] : 0.0f);
      cand[i] = ((uint64_t)f32_order_key(r) << 32) | (uint32_t)(~(uint32_t)e);
    } else {
      cand[i] = 0;
    }
  }
  uint32_t taken = 0;
  for (int round = 0; round < k; ++round) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (!((taken >> i) & 1u) && cand[i] > best) best = cand[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = shfl_xor_u64(best, off);
      best = o > best ? o : best;
    }
    const uint32_t ew = ~(uint32_t)best;
    if ((int)(ew & 63u) == lane) taken |= 1u << (ew >> 6);
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool mine = (taken >> i) & 1u;
    const uint64_t ballot = __ballot(mine);
    if (mine) {
      const int pos = base + __popcll(ballot & ((1ull << lane) - 1ull));
      const int e = lane + 64 * i;
      idx[t * k + pos] = e;
      w[t * k + pos] = sigmoid_f(zr[e]);
    }
    base += __popcll(ballot);
  }
}

hipError_t launch_topk(const float *z, const float *alpha, int64_t bt, int64_t n_experts,
                       int64_t k, int32_t *idx, float *w, hipStream_t s) {
  if (bt <= 0) return hipSuccess;
  const dim3 grid((unsigned)((bt + 3) / 4)), block(256);
  const int E = (int)n_experts, K = (int)k;
  switch ((E + 63) / 64) {
#define MOE_TOPK_CASE(n) \
  case n:                \
    return launch_kernel(topk_kernel<n>, grid, block, 0, s, z, alpha, bt, E, K, idx, w);
    MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(5) MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(9) MOE_TOPK_CASE(10) MOE_TOPK_CASE(11) MOE_TOPK_CASE(12)
    MOE_TOPK_CASE(13) MOE_TOPK_CASE(14) MOE_TOPK_CASE(15) MOE_TOPK_CASE(16)
#undef MOE_TOPK_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// ---- small fills ----------------------------------------------------------------
__global__ void copy_or_zero_f32_kernel(float *dst, const float *src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}
__global__ void zero_i32_kernel(int32_t *dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = 0;
}

hipError_t launch_copy_or_zero_f32(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return launch_kernel(copy_or_zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       dst, src, n);
}
// alpha += rate * (zeta - alpha), rounded at each step (no fused multiply-add:
// the pragma keeps the compiler from contracting the product and the sum)
__global__ void __launch_bounds__(256) cutoff_update_kernel(float *alpha, const float *zeta,
                                                            int64_t n, float rate) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const float a = alpha[i];
    const float step = rate * (zeta[i] - a);
    alpha[i] = a + step;
  }
}

hipError_t launch_cutoff_update(float *alpha, const float *zeta, int64_t n, float rate,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return launch_kernel(cutoff_update_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       alpha, zeta, n, rate);
}

hipError_t launch_zero_i32(int32_t *dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return launch_kernel(zero_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst,
                       n);
}

}  // namespace moe
