// dispatch.hip -- grouping of (token, expert) pairs by expert.
//
// On one GPU the dispatch exchange of the MoE layer (mkdocs.reaper.mx "Vue
// d'ensemble de l'architecture", section "Vérification de compréhension":
// one dispatch and one combine per MoE layer) becomes a permutation of the
// pair list into expert-contiguous segments, which GroupedExperts then runs
// as one grouped GEMM (tech.news18a.com "KimiK3的StableLatentMoE架构解析",
// figure 1: experts packed by group for memory locality).
//
// Deterministic stable counting sort, no order-dependent atomics:
//   1. per block of 64 tokens, an LDS bitmask per expert of the tokens that
//      chose it (ds_or_b64); popcounts add into counts[e] (integer sums);
//   2. one workgroup scans counts -> offsets, and ceil(counts / tile_bm) ->
//      the first M-tile of each expert for the grouped GEMMs;
//   3. one workgroup per expert walks its masks in token order: a prefix
//      over the blocks' popcounts places every pair at its stable position
//      (and, for the forward pass, copies the pair's routing weight there).
// Caller-given ids may be out of range or repeated within a token's row: such
// pairs are left out (offsets[E] < bt * k then tells), every write stays in
// its array, and inv_perm of a left-out pair is 0.  The order of the ids in a
// row does not matter.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) dispatch_mask_kernel(const int32_t *__restrict__ idx,
                                                            int64_t bt, int k, int E, int nb,
                                                            uint64_t *__restrict__ masks,
                                                            int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ inv_perm) {
  extern __shared__ uint64_t bits[];  // [E]
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) bits[e] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int ntok = (int)min((int64_t)64, bt - t0);
  for (int p = tid; p < ntok * k; p += 256) {
    const int tl = p / k, j = p - tl * k;
    const int32_t *row = idx + (t0 + tl) * k;
    const int e = row[j];
    // a pair counts when its id is in range and not repeated earlier in the
    // row; any other pair (caller-given ids only) is dropped from the
    // grouping, and its inv_perm slot is pointed at position 0 so that no
    // consumer of inv_perm reads outside the pair range
    bool ok = e >= 0 && e < E;
    for (int q = 0; q < j && ok; ++q) ok = row[q] != e;
    if (ok) atomicOr((unsigned long long *)&bits[e], 1ull << tl);
    else inv_perm[t0 * k + p] = 0;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const uint64_t m = bits[e];
    masks[(int64_t)e * nb + blockIdx.x] = m;
    const int c = __popcll(m);
    if (c) atomicAdd(&counts[e], c);
  }
}

// One workgroup of 1024 threads; E <= 1024.
__global__ void __launch_bounds__(1024) dispatch_scan_kernel(const int32_t *__restrict__ counts,
                                                             int E, int tile_bm,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ tile_offsets) {
  __shared__ int32_t wsum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t c = tid < E ? counts[tid] : 0;
  const int32_t tc = (c + tile_bm - 1) / tile_bm;
  int32_t a = c, b = tc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t oa = __shfl_up(a, off, 64), ob = __shfl_up(b, off, 64);
    if (lane >= off) { a += oa; b += ob; }
  }
  if (lane == 63) { wsum[0][wave] = a; wsum[1][wave] = b; }
  __syncthreads();
  int32_t pa = 0, pb = 0;
  for (int w = 0; w < wave; ++w) { pa += wsum[0][w]; pb += wsum[1][w]; }
  a += pa;
  b += pb;
  if (tid < E) {
    offsets[tid + 1] = a;
    tile_offsets[tid + 1] = b;
  }
  if (tid == 0) {
    offsets[0] = 0;
    tile_offsets[0] = 0;
  }
}

// Slot j of expert e in a token's row of k ids: its first occurrence (the
// mask kernel counted only that one), in any id order.
__device__ __forceinline__ int slot_of(const int32_t *row, int k, int32_t e) {
  int j = 0;
  while (j < k - 1 && row[j] != e) ++j;
  return j;
}

__global__ void __launch_bounds__(256) dispatch_scatter_kernel(
    const uint64_t *__restrict__ masks, int nb, const int32_t *__restrict__ idx, int k,
    const int32_t *__restrict__ offsets, const float *__restrict__ w,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm, float *__restrict__ w_sorted) {
  __shared__ int32_t wsum[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t *mk = masks + (int64_t)e * nb;
  int32_t run = offsets[e];
  for (int b0 = 0; b0 < nb; b0 += 256) {
    const int b = b0 + tid;
    uint64_t m = b < nb ? mk[b] : 0ull;
    const int32_t c = __popcll(m);
    int32_t incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    int32_t pos = run + before + incl - c;
    while (m) {
      const int tl = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int64_t t = (int64_t)b * 64 + tl;
      const int j = slot_of(idx + t * k, k, e);
      const int32_t p = (int32_t)(t * k + j);
      perm[pos] = p;
      inv_perm[p] = pos;
      if (w_sorted) w_sorted[pos] = w[p];
      ++pos;
    }
    run += total;
    __syncthreads();
  }
}

hipError_t launch_dispatch(const int32_t *idx, const float *w, int64_t bt, int64_t k,
                           int64_t n_experts, int tile_bm, uint64_t *masks, int32_t *counts,
                           int32_t *offsets, int32_t *tile_offsets, int32_t *perm,
                           int32_t *inv_perm, float *w_sorted, hipStream_t s) {
  const int E = (int)n_experts;
  hipError_t err = launch_zero_i32(counts, E, s);
  if (err != hipSuccess) return err;
  const int nb = (int)((bt + 63) / 64);
  if (nb > 0) {
    err = launch_kernel(dispatch_mask_kernel, dim3(nb), dim3(256), sizeof(uint64_t) * E, s, idx,
                        bt, (int)k, E, nb, masks, counts, inv_perm);
    if (err != hipSuccess) return err;
  }
  err = launch_kernel(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, counts, E, tile_bm, offsets,
                      tile_offsets);
  if (err != hipSuccess) return err;
  if (nb > 0)
    err = launch_kernel(dispatch_scatter_kernel, dim3(E), dim3(256), 0, s, masks, nb, idx, (int)k,
                        offsets, w_sorted ? w : nullptr, perm, inv_perm, w_sorted);
  return err;
}

}  // namespace moe
