// Backward pass of the Stable LatentMoE layer (bf16 activations and weights).
//
// The pages give the forward pass (tech.news18a.com page: the architecture
// figure, the SiTU formula, the "quantile balancing" passage); the training
// motivation of its caps and cutoffs is the same page's gradient-explosion
// passage.  The gradients are the chain rule of that forward:
//   * the chosen expert set is piecewise constant in the scores and carries no
//     gradient; a chosen pair's weight w = sigmoid(z) does: dz = dw w (1 - w);
//   * h = w phi(g) psi(u), o = W_d h, y_lat = sum of o, n = y_lat r gamma,
//     y = W_up n + sum_s W_ds,s hs_s, hs = phi(W_gs x) psi(W_us x).
//
// The forward quantities the gradients need (x_lat, each pair's g and u, h,
// o, y_lat and r, the shared experts' g and u) are recomputed here from x and
// the routing that moe_route returned, so a caller keeps no activations.
// Every contraction runs on the layer's GEMM engine, in one of three forms:
// the forward's ([M][K] x [N][K]), the input gradients' (the weight operand
// read K-outer, as stored: dx = dy W), and the weight gradients' (both
// operands K-outer, K = tokens; for the routed experts one output per expert
// over its pairs).  The routed experts' contractions are grouped by expert
// from the dispatch offsets on the device, one launch each: nothing waits for
// the host.  Every elementwise step, gather, reduction and normalisation runs
// in the kernels below.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "gemm_launch.h"
#include "kernels.h"
#include "moe.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kColChunk = 128;  // rows a partial column sum covers

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct BwdPlan {
  size_t masks, counts, offsets, tile_offsets, perm, inv_perm, w_sorted, xlat, xg, G, U, h, o,
      ylat, rinv, n, Gs, Us, hs, dn, dylat, dyg, dh, dg, du, dz, dz16, dxg, dxlat, dhs, dgs, dus,
      part, split, total;
  int64_t e_pad = 0;      // router gradient columns, padded to the K tile (zeros past E)
  int64_t split_cap = 0;  // floats of split-K partial sums (short batches)
};

bool backward_supported(const moe_config *c) {
  if (!c || c->d <= 0 || c->latent <= 0 || c->n_experts <= 0 || c->n_experts > 1024 ||
      c->top_k <= 0 || c->top_k > c->n_experts || c->top_k > 64 || c->expert_inter <= 0 ||
      c->n_shared < 0 || c->n_shared > 4 || (c->n_shared > 0 && c->shared_inter <= 0))
    return false;
  return true;
}

moe_status bwd_plan(const moe_config *c, int64_t bt, BwdPlan *p) {
  if (!backward_supported(c) || bt < 0) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_BF16 || c->weight_dtype != MOE_BF16 || c->router_dtype != MOE_BF16)
    return MOE_ERR_UNSUPPORTED;
  // the engine's K tiles (64) over d, L, I and I_s as K of stored operands;
  // 16-byte rows chunks of K-outer operands (E columns of the router gradient)
  if (c->d % 64 || c->latent % 64 || c->expert_inter % 64 ||
      (c->n_shared && c->shared_inter % 64) || c->n_experts % 8)
    return MOE_ERR_UNSUPPORTED;
  const int64_t E = c->n_experts, L = c->latent, I = c->expert_inter, d = c->d;
  const int64_t SI = c->n_shared * c->shared_inter, P = bt * c->top_k;
  // 32-bit element counts in the kernels; gathered rows addressed with 32-bit offsets
  if (P >= (int64_t)1 << 31 || P * std::max(L, I) >= (int64_t)1 << 31 ||
      bt * std::max({d, L, E, SI}) >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  const int64_t nb = (bt + 63) / 64, nchunk = (bt + kColChunk - 1) / kColChunk;
  p->e_pad = (E + 63) / 64 * 64;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    size_t o = off;
    off += align_up((size_t)bytes);
    return o;
  };
  p->masks = take(8 * E * nb);
  p->counts = take(4 * E);
  p->offsets = take(4 * (E + 1));
  p->tile_offsets = take(4 * (E + 1));
  p->perm = take(4 * P);
  p->inv_perm = take(4 * P);
  p->w_sorted = take(4 * P);
  p->xlat = take(2 * bt * L);
  p->xg = take(2 * P * L);
  p->G = take(4 * P * I);
  p->U = take(4 * P * I);
  p->h = take(2 * P * I);
  p->o = take(2 * P * L);
  p->ylat = take(4 * bt * L);
  p->rinv = take(4 * bt);
  p->n = take(2 * bt * L);
  p->Gs = take(4 * bt * SI);
  p->Us = take(4 * bt * SI);
  p->hs = take(2 * bt * SI);
  p->dn = take(4 * bt * L);
  p->dylat = take(2 * bt * L);
  p->dyg = take(2 * P * L);
  p->dh = take(4 * P * I);
  p->dg = take(2 * P * I);
  p->du = take(2 * P * I);
  p->dz = take(4 * bt * E);
  p->dz16 = take(2 * bt * p->e_pad);
  p->dxg = take(4 * P * L);
  p->dxlat = take(2 * bt * L);
  p->dhs = take(4 * bt * SI);
  p->dgs = take(2 * bt * SI);
  p->dus = take(2 * bt * SI);
  p->part = take(4 * nchunk * std::max(L, E));
  // split-K partial sums of the dense input-gradient GEMMs of short batches
  if (bt > 0 && bt <= 256) p->split_cap = 16 * bt * std::max({d, L, SI, E});
  p->split = take(4 * p->split_cap);
  p->total = off;
  return MOE_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

#define MOE_TRY(expr)                            \
  do {                                           \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)
// ---- elementwise and reduction kernels ------------------------------------------------
struct Situ {
  float phi, dphi, psi, dpsi;
};
// phi(g) = s beta tanh(g / beta) with s = sigmoid(g):
//   phi' = s (1 - s) beta tanh(g / beta) + s (1 - tanh^2(g / beta));
// psi(u) = beta_u tanh(u / beta_u): psi' = 1 - tanh^2(u / beta_u).
__device__ __forceinline__ Situ situ_parts(float g, float u, float beta, float inv_beta,
                                           float beta_u, float inv_beta_u) {
  const float s = sigmoid_f(g);
  const float tg = tanh_f(g * inv_beta);
  const float tu = tanh_f(u * inv_beta_u);
  Situ r;
  r.phi = s * beta * tg;
  r.dphi = s * (1.0f - s) * beta * tg + s * (1.0f - tg * tg);
  r.psi = beta_u * tu;
  r.dpsi = 1.0f - tu * tu;
  return r;
}

// dst[q][:] = src[perm[q] / k][:] (bf16 rows, 8 values a thread) for the rows
// q < *rows_end (the dispatched pairs)
__global__ void gather_rows_kernel(const uint16_t *__restrict__ src,
                                   const int32_t *__restrict__ perm, int k, int64_t rows,
                                   int64_t cols, const int32_t *__restrict__ rows_end,
                                   uint16_t *__restrict__ dst) {
  const int64_t c8 = cols / 8, n = rows * c8, q_end = *rows_end;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = i / c8, c = i % c8;
    if (q >= q_end) continue;
    const int64_t t = perm[q] / k;
    reinterpret_cast<uint4 *>(dst + q * cols)[c] =
        reinterpret_cast<const uint4 *>(src + t * cols)[c];
  }
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// One block a token: y_lat = sum_j o[inv_perm[t k + j]] (j ascending), r = (mean y_lat^2 +
// eps)^(-1/2), n = bf16(y_lat r gamma).
__global__ void combine_ylat_kernel(const uint16_t *__restrict__ o,
                                    const int32_t *__restrict__ inv_perm, int k, int64_t L,
                                    const float *__restrict__ gamma, float eps,
                                    float *__restrict__ ylat, float *__restrict__ rinv,
                                    uint16_t *__restrict__ n) {
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  float ss = 0.0f;
  for (int64_t l = threadIdx.x; l < L; l += blockDim.x) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc += bf16_to_f32(o[(int64_t)inv_perm[t * k + j] * L + l]);
    ylat[t * L + l] = acc;
    ss += acc * acc;
  }
  const float r = 1.0f / sqrtf(block_sum(ss, red) / (float)L + eps);
  if (threadIdx.x == 0) rinv[t] = r;
  for (int64_t l = threadIdx.x; l < L; l += blockDim.x)
    n[t * L + l] = f32_to_bf16(ylat[t * L + l] * r * gamma[l]);
}

// One block a token: dy_lat = r gamma dn - y_lat r^3 (sum_l gamma dn y_lat) / L -> bf16
__global__ void rms_bwd_kernel(const float *__restrict__ dn, const float *__restrict__ ylat,
                               const float *__restrict__ rinv, const float *__restrict__ gamma,
                               int64_t L, uint16_t *__restrict__ dylat) {
  __shared__ float red[16];
  const int64_t t = blockIdx.x;
  const float *dr = dn + t * L, *yr = ylat + t * L;
  float s = 0.0f;
  for (int64_t l = threadIdx.x; l < L; l += blockDim.x) s += gamma[l] * dr[l] * yr[l];
  s = block_sum(s, red);
  const float r = rinv[t], c = r * r * r * s / (float)L;
  for (int64_t l = threadIdx.x; l < L; l += blockDim.x)
    dylat[t * L + l] = f32_to_bf16(r * gamma[l] * dr[l] - yr[l] * c);
}

// Partial column sums over chunks of kColChunk rows: part[chunk][c] =
// sum_r a[r][c] * (b ? b[r][c] : 1) * (rs ? rs[r] : 1).
__global__ void colsum_part_kernel(const float *__restrict__ a, const float *__restrict__ b,
                                   const float *__restrict__ rs, int64_t rows, int64_t cols,
                                   float *__restrict__ part) {
  const int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (c >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * kColChunk, r1 = std::min(rows, r0 + kColChunk);
  float acc = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    float v = a[r * cols + c];
    if (b) v *= b[r * cols + c];
    if (rs) v *= rs[r];
    acc += v;
  }
  part[(int64_t)blockIdx.y * cols + c] = acc;
}
__global__ void colsum_final_kernel(const float *__restrict__ part, int64_t nchunk, int64_t cols,
                                    float *__restrict__ out) {
  const int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float acc = 0.0f;
  for (int64_t i = 0; i < nchunk; ++i) acc += part[i * cols + c];
  out[c] = acc;
}

// One wave a row q: dg = dh w psi phi', du = dh w phi psi' (bf16), dw = sum dh phi psi;
// with dz, dz[t][e] = dw w (1 - w) for the pair p = perm[q] (t = p / k, e = idx[p]).
// w = NULL: weight 1 and no dz (the shared experts).
__global__ void situ_bwd_kernel(const float *__restrict__ dh, const float *__restrict__ G,
                                const float *__restrict__ U, const float *__restrict__ w,
                                const int32_t *__restrict__ perm,
                                const int32_t *__restrict__ idx, int k, int64_t E, int64_t rows,
                                int64_t cols, const int32_t *__restrict__ rows_end, float beta,
                                float inv_beta, float beta_u, float inv_beta_u,
                                uint16_t *__restrict__ dg, uint16_t *__restrict__ du,
                                float *__restrict__ dz) {
  const int lane = threadIdx.x & 63;
  const int64_t q = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (q >= rows || (rows_end && q >= *rows_end)) return;
  const float wq = w ? w[q] : 1.0f;
  float dw = 0.0f;
  for (int64_t i = lane; i < cols; i += 64) {
    const int64_t x = q * cols + i;
    const Situ s = situ_parts(G[x], U[x], beta, inv_beta, beta_u, inv_beta_u);
    const float d = dh[x];
    dw += d * (s.phi * s.psi);
    dg[x] = f32_to_bf16(d * wq * s.psi * s.dphi);
    du[x] = f32_to_bf16(d * wq * s.phi * s.dpsi);
  }
  if (!dz) return;
  for (int o = 32; o > 0; o >>= 1) dw += __shfl_xor(dw, o);
  if (lane == 0) {
    const int64_t p = perm[q];
    dz[(p / k) * E + idx[p]] = dw * wq * (1.0f - wq);
  }
}

// dst[t][:] = bf16(sum_j src[inv_perm[t k + j]][:]) (j ascending)
__global__ void combine_rows_kernel(const float *__restrict__ src,
                                    const int32_t *__restrict__ inv_perm, int k, int64_t bt,
                                    int64_t L, uint16_t *__restrict__ dst) {
  const int64_t n = bt * L;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / L, l = i % L;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc += src[(int64_t)inv_perm[t * k + j] * L + l];
    dst[i] = f32_to_bf16(acc);
  }
}

__global__ void fill_f32_kernel(float *__restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}
// d[r][c] = bf16(s[r][c]) for c < cols, 0 for cols <= c < ld
__global__ void cvt_bf16_pad_kernel(const float *__restrict__ s, int64_t rows, int64_t cols,
                                    int64_t ld, uint16_t *__restrict__ d) {
  const int64_t n = rows * ld;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ld, c = i % ld;
    d[i] = c < cols ? f32_to_bf16(s[r * cols + c]) : (uint16_t)0;
  }
}

// grid-stride launches: at most 65536 blocks of 256
dim3 grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 65536)));
}

hipError_t fill_f32(float *p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch_kernel(fill_f32_kernel, grid_for(n), dim3(256), 0, s, p, n);
}

hipError_t colsum(const float *a, const float *b, const float *rs, int64_t rows, int64_t cols,
                  float *part, float *out, hipStream_t s) {
  const int64_t nchunk = (rows + kColChunk - 1) / kColChunk;
  if (nchunk == 0) return fill_f32(out, cols, s);
  const dim3 g((unsigned)((cols + 255) / 256), (unsigned)nchunk);
  hipError_t e = launch_kernel(colsum_part_kernel, g, dim3(256), 0, s, a, b, rs, rows, cols, part);
  if (e != hipSuccess) return e;
  return launch_kernel(colsum_final_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, s,
                       (const float *)part, nchunk, cols, out);
}

// ---- contractions on the GEMM engine ---------------------------------------------------
// One contraction C = op(A) op(B) with fp32 output (the recomputations keep
// the forward's bf16 kinds): A [M][K] as stored or K-outer [K][M], B [N][K]
// or K-outer [K][N].
struct Contraction {
  GemmArgs a = {};
  Contraction(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
              int64_t ldb, void *C, int64_t ldc) {
    a.M = M;
    a.N = N;
    a.nseg = 1;
    a.seg[0] = GemmSeg{A, lda, B, ldb, nullptr, K};
    a.out = C;
    a.ldo = ldc;
    a.beta = a.inv_beta = a.beta_u = a.inv_beta_u = 1.0f;
  }
  // grouped by expert: rows offsets[e].. of A against expert e's B
  Contraction &by_expert(const int32_t *offsets, const int32_t *tile_offsets, int64_t E,
                         int64_t b_estride) {
    a.offsets = offsets;
    a.tile_offsets = tile_offsets;
    a.n_experts = (int32_t)E;
    a.b_estride = b_estride;
    return *this;
  }
  // C = A B + A1 B1 (B K-outer, grouped): a second K segment with A's and B's
  // strides and K (whole K tiles), in the same launch
  Contraction &and_(const void *A1, const void *B1) {
    a.nseg = 2;
    a.seg[1] = GemmSeg{A1, a.seg[0].lda, B1, a.seg[0].ldb, nullptr, a.seg[0].k};
    return *this;
  }
  Contraction &plus(const float *c_in) {  // C = c_in + op(A) op(B) (c_in may be C)
    a.resid = c_in;
    a.ldr = a.ldo;
    return *this;
  }
  Contraction &split(float *partial, int64_t cap) {  // short batches: split K
    a.partial = partial;
    a.partial_cap = cap;
    return *this;
  }
};

// C = A B^T, fp32 (the stored layouts; dense or grouped)
hipError_t nt_f32(const Contraction &c, int v, hipStream_t s) {
  return launch_dma<EPI_STORE, false, false, float, false>(v, c.a, s);
}
// C = A B with B K-outer ([K][N], per expert when grouped): input gradients
// (two K segments: grouped, unsplit, whole 64-wide K tiles)
hipError_t nn_f32(const Contraction &c, int v, hipStream_t s) {
  if (c.a.nseg == 2 && (c.a.offsets == nullptr || c.a.partial != nullptr || c.a.seg[0].k % 64 ||
                        c.a.seg[1].k != c.a.seg[0].k))
    return hipErrorInvalidValue;
  return launch_dma_ko<EPI_STORE, false, true, false, false, float>(v, c.a, s);
}
// C = A^T B with both operands K-outer (K = tokens): dense weight gradients
hipError_t tn_f32(const Contraction &c, hipStream_t s) {
  return launch_dma_ko<EPI_STORE, true, true, false, false, float>(kVDense, c.a, s);
}
// C_e = A_e^T B_e over the rows offsets[e].. of both: the routed experts' weight gradients
hipError_t tn_experts_f32(Contraction c, const int32_t *offsets, int64_t E, hipStream_t s) {
  c.a.offsets = offsets;
  c.a.n_experts = (int32_t)E;
  return launch_dma_ko<EPI_STORE, true, true, true, false, float>(kgrp_variant(), c.a, s);
}

GemmArgs base_args_bwd(const moe_config *c) {
  GemmArgs a = {};
  a.beta = c->beta;
  a.inv_beta = 1.0f / c->beta;
  a.beta_u = c->beta_u;
  a.inv_beta_u = 1.0f / c->beta_u;
  return a;
}

bool grads_complete(const moe_config *c, const moe_grads *g, int64_t bt) {
  return g && (g->dx || bt == 0) && g->w_router && g->router_bias && g->w_down_proj && g->w_gate &&
         g->w_up && g->w_down && g->latent_gamma && g->w_up_proj &&
         (c->n_shared == 0 || (g->sh_gate && g->sh_up && g->sh_down));
}

}  // namespace

MOE_API size_t moe_backward_workspace_bytes(const moe_config *cfg, int64_t bt) {
  BwdPlan p;
  if (bwd_plan(cfg, bt, &p) != MOE_OK) return 0;
  return p.total;
}

MOE_API moe_status moe_backward(const moe_config *cfg, const moe_weights *w, const void *x,
                                int64_t bt, const int32_t *topk_idx, const float *topk_w,
                                const void *dy, const moe_grads *g, void *ws, size_t ws_bytes,
                                void *stream) {
  BwdPlan p;
  moe_status st = bwd_plan(cfg, bt, &p);
  if (st != MOE_OK) return st;
  if (!w || !grads_complete(cfg, g, bt)) return MOE_ERR_INVALID_ARG;
  if (!w->w_router || !w->w_down_proj || !w->w_gate || !w->w_up || !w->w_down ||
      !w->w_up_proj || (cfg->n_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)))
    return MOE_ERR_INVALID_ARG;
  if (w->expert_tab) return MOE_ERR_UNSUPPORTED;
  if (bt > 0 && (!x || !topk_idx || !topk_w || !dy)) return MOE_ERR_INVALID_ARG;
  if (bt > 0 && (!ws || ws_bytes < p.total || reinterpret_cast<uintptr_t>(ws) % kAlign))
    return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t d = cfg->d, L = cfg->latent, E = cfg->n_experts, k = cfg->top_k;
  const int64_t I = cfg->expert_inter, S = cfg->n_shared, Is = cfg->shared_inter, SI = S * Is;
  const int64_t P = bt * k;
  if (bt == 0) {  // every gradient is zero
    const std::pair<float *, int64_t> all[] = {
        {g->w_router, E * d}, {g->router_bias, E}, {g->w_down_proj, L * d},
        {g->w_gate, E * I * L}, {g->w_up, E * I * L}, {g->w_down, E * L * I},
        {g->latent_gamma, L}, {g->w_up_proj, d * L}, {g->sh_gate, SI * d},
        {g->sh_up, SI * d}, {g->sh_down, S * d * Is}};
    for (const auto &a : all)
      if (a.first) MOE_TRY(fill_f32(a.first, a.second, s));
    return MOE_OK;
  }
  const float beta = cfg->beta, ib = 1.0f / cfg->beta, bu = cfg->beta_u, ibu = 1.0f / cfg->beta_u;

  int32_t *counts = at<int32_t>(ws, p.counts), *offsets = at<int32_t>(ws, p.offsets);
  int32_t *tile_offsets = at<int32_t>(ws, p.tile_offsets);
  int32_t *perm = at<int32_t>(ws, p.perm), *inv_perm = at<int32_t>(ws, p.inv_perm);
  float *w_sorted = at<float>(ws, p.w_sorted);
  uint16_t *xlat = at<uint16_t>(ws, p.xlat), *xg = at<uint16_t>(ws, p.xg);
  float *G = at<float>(ws, p.G), *U = at<float>(ws, p.U);
  uint16_t *h = at<uint16_t>(ws, p.h), *o = at<uint16_t>(ws, p.o), *n = at<uint16_t>(ws, p.n);
  float *ylat = at<float>(ws, p.ylat), *rinv = at<float>(ws, p.rinv);
  float *Gs = at<float>(ws, p.Gs), *Us = at<float>(ws, p.Us);
  uint16_t *hs = at<uint16_t>(ws, p.hs);
  float *dn = at<float>(ws, p.dn), *dh = at<float>(ws, p.dh), *dz = at<float>(ws, p.dz);
  uint16_t *dylat = at<uint16_t>(ws, p.dylat), *dyg = at<uint16_t>(ws, p.dyg);
  uint16_t *dg = at<uint16_t>(ws, p.dg), *du = at<uint16_t>(ws, p.du);
  uint16_t *dz16 = at<uint16_t>(ws, p.dz16), *dxlat = at<uint16_t>(ws, p.dxlat);
  float *dxg = at<float>(ws, p.dxg), *dhs = at<float>(ws, p.dhs), *part = at<float>(ws, p.part);
  float *split = at<float>(ws, p.split);
  uint16_t *dgs = at<uint16_t>(ws, p.dgs), *dus = at<uint16_t>(ws, p.dus);
  const int32_t *pairs_end = offsets + E;  // dispatched pairs (bt k for valid routing)
  // tile shapes: the routed experts' GEMMs as the forward's, short batches' dense ones
  const int vg = dma_variant(GK_EXPERT_SITU, P, E);
  const int vd = bt <= 64 ? kVSmallM : kVDense;
  const int64_t dense_mt = (bt + gemm_bm(PATH_BF16) - 1) / gemm_bm(PATH_BF16);
  const int64_t grouped_mt = (P + gemm_bm(PATH_BF16) - 1) / gemm_bm(PATH_BF16) + E;

  // ---- recompute: dispatch, x_lat, the routed experts, y_lat and r -------------------
  MOE_TRY(launch_dispatch(topk_idx, topk_w, bt, k, E, grouped_tile_rows(PATH_BF16, WF_BF16, P, E),
                          at<uint64_t>(ws, p.masks), counts, offsets, tile_offsets, perm,
                          inv_perm, w_sorted, s));
  {
    GemmArgs a = base_args_bwd(cfg);
    a.M = bt;
    a.N = L;
    a.nseg = 1;
    a.seg[0] = GemmSeg{x, d, w->w_down_proj, d, nullptr, d};
    a.out = xlat;
    a.ldo = L;
    a.partial = split;
    a.partial_cap = p.split_cap;
    MOE_TRY(gemm_launch(a, PATH_BF16, GK_DENSE, WF_BF16, dense_mt, s));
  }
  MOE_TRY(launch_kernel(gather_rows_kernel, grid_for(P * L / 8), dim3(256), 0, s,
                        (const uint16_t *)xlat, (const int32_t *)perm, (int)k, P, L, pairs_end,
                        xg));
  {
    // the forward's gate/up launch (gathered rows, h = w phi(g) psi(u)), also
    // writing each pair's raw g and u in fp32
    GemmArgs a = base_args_bwd(cfg);
    a.M = P;
    a.N = I;
    a.nseg = 1;
    a.seg[0] = GemmSeg{xlat, L, w->w_gate, L, nullptr, L};
    a.b_up = w->w_up;
    a.offsets = offsets;
    a.tile_offsets = tile_offsets;
    a.n_experts = (int32_t)E;
    a.b_estride = I * L;
    a.gather = perm;
    a.gather_div = (int32_t)k;
    a.row_scale = w_sorted;
    a.out = h;
    a.ldo = I;
    a.out_g = G;
    a.out_u = U;
    a.ldgu = I;
    MOE_TRY(gemm_launch(a, PATH_BF16, GK_EXPERT_SITU, WF_BF16, grouped_mt, s));
  }
  {
    GemmArgs a = base_args_bwd(cfg);
    a.M = P;
    a.N = L;
    a.nseg = 1;
    a.seg[0] = GemmSeg{h, I, w->w_down, I, nullptr, I};
    a.offsets = offsets;
    a.tile_offsets = tile_offsets;
    a.n_experts = (int32_t)E;
    a.b_estride = L * I;
    a.out = o;
    a.ldo = L;
    MOE_TRY(gemm_launch(a, PATH_BF16, GK_EXPERT_DOWN, WF_BF16, grouped_mt, s));
  }
  MOE_TRY(launch_kernel(combine_ylat_kernel, dim3((unsigned)bt), dim3(256), 0, s,
                        (const uint16_t *)o, (const int32_t *)inv_perm, (int)k, L,
                        w->latent_gamma, cfg->rms_eps, ylat, rinv, n));
  if (S > 0) {  // the S shared experts' gate / up rows are one [S I_s][d] matrix each
    // the forward's shared gate/up launch, also writing the raw g and u
    GemmArgs a = base_args_bwd(cfg);
    a.M = bt;
    a.N = SI;
    a.nseg = 1;
    a.seg[0] = GemmSeg{x, d, w->sh_gate, d, nullptr, d};
    a.b_up = w->sh_up;
    a.partial = split;
    a.partial_cap = p.split_cap;
    a.out = hs;
    a.ldo = SI;
    a.out_g = Gs;
    a.out_u = Us;
    a.ldgu = SI;
    MOE_TRY(gemm_launch(a, PATH_BF16, GK_DENSE_SITU, WF_BF16, dense_mt, s));
  }

  // ---- y = W_up n + sum_s W_ds,s hs_s ----------------------------------------------
  MOE_TRY(tn_f32(Contraction(d, L, bt, dy, d, n, L, g->w_up_proj, L), s));
  MOE_TRY(nn_f32(Contraction(bt, L, d, dy, d, w->w_up_proj, L, dn, L).split(split, p.split_cap),
                 vd, s));
  const uint16_t *shd = static_cast<const uint16_t *>(w->sh_down);
  for (int64_t sx = 0; sx < S; ++sx) {
    MOE_TRY(tn_f32(Contraction(d, Is, bt, dy, d, hs + sx * Is, SI, g->sh_down + sx * d * Is, Is), s));
    MOE_TRY(nn_f32(Contraction(bt, Is, d, dy, d, shd + sx * d * Is, Is, dhs + sx * Is, SI)
                       .split(split, p.split_cap), vd, s));
  }
  // ---- n = y_lat r gamma ------------------------------------------------------------
  MOE_TRY(colsum(dn, ylat, rinv, bt, L, part, g->latent_gamma, s));
  MOE_TRY(launch_kernel(rms_bwd_kernel, dim3((unsigned)bt), dim3(256), 0, s, (const float *)dn,
                        (const float *)ylat, (const float *)rinv, w->latent_gamma, L, dylat));
  // ---- routed experts ---------------------------------------------------------------
  MOE_TRY(launch_kernel(gather_rows_kernel, grid_for(P * L / 8), dim3(256), 0, s,
                        (const uint16_t *)dylat, (const int32_t *)perm, (int)k, P, L, pairs_end,
                        dyg));
  // dW_d,e = dy_e^T h_e over expert e's pairs (zero for an expert no pair chose)
  MOE_TRY(tn_experts_f32(Contraction(L, I, 0, dyg, L, h, I, g->w_down, I), offsets, E, s));
  MOE_TRY(nn_f32(Contraction(P, I, L, dyg, L, w->w_down, I, dh, I)
                     .by_expert(offsets, tile_offsets, E, L * I), vg, s));
  MOE_TRY(fill_f32(dz, bt * E, s));
  MOE_TRY(launch_kernel(situ_bwd_kernel, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, s,
                        (const float *)dh, (const float *)G, (const float *)U,
                        (const float *)w_sorted, (const int32_t *)perm, topk_idx, (int)k, E, P,
                        I, pairs_end, beta, ib, bu, ibu, dg, du, dz));
  MOE_TRY(tn_experts_f32(Contraction(I, L, 0, dg, I, xg, L, g->w_gate, L), offsets, E, s));
  MOE_TRY(tn_experts_f32(Contraction(I, L, 0, du, I, xg, L, g->w_up, L), offsets, E, s));
  // dx_lat rows = dg W_g + du W_u: one launch over both K segments
  MOE_TRY(nn_f32(Contraction(P, L, I, dg, I, w->w_gate, L, dxg, L)
                     .by_expert(offsets, tile_offsets, E, I * L)
                     .and_(du, w->w_up), vg, s));
  MOE_TRY(launch_kernel(combine_rows_kernel, grid_for(bt * L), dim3(256), 0, s,
                        (const float *)dxg, (const int32_t *)inv_perm, (int)k, bt, L, dxlat));
  // ---- x_lat = W_down_proj x, and the router ------------------------------------------
  MOE_TRY(tn_f32(Contraction(L, d, bt, dxlat, L, x, d, g->w_down_proj, d), s));
  MOE_TRY(nn_f32(Contraction(bt, d, L, dxlat, L, w->w_down_proj, d, g->dx, d)
                     .split(split, p.split_cap), vd, s));
  MOE_TRY(launch_kernel(cvt_bf16_pad_kernel, grid_for(bt * p.e_pad), dim3(256), 0, s,
                        (const float *)dz, bt, E, p.e_pad, dz16));
  MOE_TRY(tn_f32(Contraction(E, d, bt, dz16, p.e_pad, x, d, g->w_router, d), s));
  // (K = E: the router rows past E are masked, the padded dz columns are zero)
  MOE_TRY(nn_f32(Contraction(bt, d, E, dz16, p.e_pad, w->w_router, d, g->dx, d)
                     .plus(g->dx).split(split, p.split_cap), vd, s));
  MOE_TRY(colsum(dz, nullptr, nullptr, bt, E, part, g->router_bias, s));
  // ---- shared experts ---------------------------------------------------------------
  if (S > 0) {
    MOE_TRY(launch_kernel(situ_bwd_kernel, dim3((unsigned)((bt + 3) / 4)), dim3(256), 0, s,
                          (const float *)dhs, (const float *)Gs, (const float *)Us,
                          (const float *)nullptr, (const int32_t *)nullptr,
                          (const int32_t *)nullptr, 1, E, bt, SI, (const int32_t *)nullptr, beta,
                          ib, bu, ibu, dgs, dus, (float *)nullptr));
    MOE_TRY(tn_f32(Contraction(SI, d, bt, dgs, SI, x, d, g->sh_gate, d), s));
    MOE_TRY(tn_f32(Contraction(SI, d, bt, dus, SI, x, d, g->sh_up, d), s));
    MOE_TRY(nn_f32(Contraction(bt, d, SI, dgs, SI, w->sh_gate, d, g->dx, d)
                       .plus(g->dx).split(split, p.split_cap), vd, s));
    MOE_TRY(nn_f32(Contraction(bt, d, SI, dus, SI, w->sh_up, d, g->dx, d)
                       .plus(g->dx).split(split, p.split_cap), vd, s));
  }
  return MOE_OK;
}
