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
// the routing that moe_route returned, so a caller keeps no activations.  The
// contractions are plain GEMMs with transposed operands and run on rocBLAS
// (bf16 inputs, fp32 accumulation); the routed experts' GEMMs are issued per
// expert from the dispatch counts, which the call copies to the host, over
// four side streams.  Every
// elementwise step, gather, reduction and normalisation runs in the kernels
// below.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <thread>
#include <vector>

#include "common.h"
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
      part, total;
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
  // the row gathers move 8 bf16 values a thread; rocBLAS takes 32-bit sizes
  if (c->d % 8 || c->latent % 8 || c->expert_inter % 8 || c->shared_inter % 8)
    return MOE_ERR_UNSUPPORTED;
  const int64_t E = c->n_experts, L = c->latent, I = c->expert_inter, d = c->d;
  const int64_t SI = c->n_shared * c->shared_inter, P = bt * c->top_k;
  if (P >= (int64_t)1 << 31 || P * std::max(L, I) >= (int64_t)1 << 31 ||
      bt * std::max({d, L, E, SI}) >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  const int64_t nb = (bt + 63) / 64, nchunk = (bt + kColChunk - 1) / kColChunk;
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
  p->dz16 = take(2 * bt * E);
  p->dxg = take(4 * P * L);
  p->dxlat = take(2 * bt * L);
  p->dhs = take(4 * bt * SI);
  p->dgs = take(2 * bt * SI);
  p->dus = take(2 * bt * SI);
  p->part = take(4 * nchunk * std::max(L, E));
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
#define MOE_TRY_BLAS(expr)                                     \
  do {                                                         \
    if ((expr) != rocblas_status_success) return MOE_ERR_HIP; \
  } while (0)

// ---- rocBLAS and the expert streams ---------------------------------------------------
// One expert's GEMM (a few hundred rows at prefill, a few at decode) covers a
// small part of the 256 CUs, so consecutive experts go round-robin to kSide
// streams and run side by side.  Per device, created on first use with that
// device current: a handle for the caller's stream, and a stream + handle +
// event for each side; all at the default priority.
constexpr int kSide = 4;
struct Blas {
  rocblas_handle main = nullptr;
  rocblas_handle side[kSide] = {};
  hipStream_t ss[kSide] = {};
  hipEvent_t done[kSide] = {};
  hipEvent_t fork = nullptr;
  bool ok = false;
};

Blas *blas() {
  static std::mutex mu;
  static Blas per_dev[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  Blas &b = per_dev[dev];
  if (!b.ok) {
    if (!b.main && rocblas_create_handle(&b.main) != rocblas_status_success) return nullptr;
    if (!b.fork && hipEventCreateWithFlags(&b.fork, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    for (int i = 0; i < kSide; ++i) {
      if (!b.ss[i] && hipStreamCreateWithFlags(&b.ss[i], hipStreamNonBlocking) != hipSuccess)
        return nullptr;
      if (!b.done[i] && hipEventCreateWithFlags(&b.done[i], hipEventDisableTiming) != hipSuccess)
        return nullptr;
      if (!b.side[i]) {
        if (rocblas_create_handle(&b.side[i]) != rocblas_status_success) return nullptr;
        if (rocblas_set_stream(b.side[i], b.ss[i]) != rocblas_status_success) return nullptr;
      }
    }
    b.ok = true;
  }
  return &b;
}

// the side streams start after the work enqueued on s so far ...
hipError_t fork_sides(const Blas &b, hipStream_t s) {
  hipError_t e = hipEventRecord(b.fork, s);
  for (int i = 0; i < kSide && e == hipSuccess; ++i) e = hipStreamWaitEvent(b.ss[i], b.fork, 0);
  return e;
}
// ... and s continues after everything enqueued on them
hipError_t join_sides(const Blas &b, hipStream_t s) {
  hipError_t e = hipSuccess;
  for (int i = 0; i < kSide && e == hipSuccess; ++i) {
    e = hipEventRecord(b.done[i], b.ss[i]);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, b.done[i], 0);
  }
  return e;
}

// Row-major C[M][N] = op(A) op(B) + beta C with op(A) [M][K], op(B) [K][N]; ta / tb
// mean A is stored [K][M] / B is stored [N][K].  rocBLAS is column-major, where
// the row-major C is C^T = op(B)^T op(A)^T: the operands swap and keep their flags.
rocblas_status gemm_rm(rocblas_handle hd, bool ta, bool tb, int64_t M, int64_t N, int64_t K,
                       const void *A, rocblas_datatype at_, int64_t lda, const void *B,
                       rocblas_datatype bt_, int64_t ldb, float beta, void *C,
                       rocblas_datatype ct, int64_t ldc) {
  if (M == 0 || N == 0) return rocblas_status_success;
  const float alpha = 1.0f;
  return rocblas_gemm_ex(hd, tb ? rocblas_operation_transpose : rocblas_operation_none,
                         ta ? rocblas_operation_transpose : rocblas_operation_none, (int)N,
                         (int)M, (int)K, &alpha, B, bt_, (int)ldb, A, at_, (int)lda, &beta, C,
                         ct, (int)ldc, C, ct, (int)ldc, rocblas_datatype_f32_r,
                         rocblas_gemm_algo_standard, 0, 0);
}
constexpr rocblas_datatype BF = rocblas_datatype_bf16_r, F32 = rocblas_datatype_f32_r;

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

// dst[q][:] = src[perm[q] / k][:] (bf16 rows, 8 values a thread)
__global__ void gather_rows_kernel(const uint16_t *__restrict__ src,
                                   const int32_t *__restrict__ perm, int k, int64_t rows,
                                   int64_t cols, uint16_t *__restrict__ dst) {
  const int64_t c8 = cols / 8, n = rows * c8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = i / c8, c = i % c8;
    const int64_t t = perm[q] / k;
    reinterpret_cast<uint4 *>(dst + q * cols)[c] =
        reinterpret_cast<const uint4 *>(src + t * cols)[c];
  }
}

// h[q][i] = bf16(w_q phi(g) psi(u)); w = NULL: weight 1
__global__ void situ_h_kernel(const float *__restrict__ G, const float *__restrict__ U,
                              const float *__restrict__ w, int64_t rows, int64_t cols,
                              float beta, float inv_beta, float beta_u, float inv_beta_u,
                              uint16_t *__restrict__ h) {
  const int64_t n = rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const Situ s = situ_parts(G[i], U[i], beta, inv_beta, beta_u, inv_beta_u);
    const float wq = w ? w[i / cols] : 1.0f;
    h[i] = f32_to_bf16(wq * (s.phi * s.psi));
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
                                int64_t cols, float beta, float inv_beta, float beta_u,
                                float inv_beta_u, uint16_t *__restrict__ dg,
                                uint16_t *__restrict__ du, float *__restrict__ dz) {
  const int lane = threadIdx.x & 63;
  const int64_t q = blockIdx.x * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);
  if (q >= rows) return;
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
__global__ void cvt_bf16_kernel(const float *__restrict__ s, int64_t n, uint16_t *__restrict__ d) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    d[i] = f32_to_bf16(s[i]);
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

// Runs fn(e, handle, stream) for every expert e, expert e on side e % kSide;
// each side's experts are issued by a host thread of its own (a library call
// per GEMM costs microseconds of host time, comparable to a small expert's
// GEMM).  The sides start after the work on s so far, and s waits for them.
template <typename Fn>
moe_status for_experts(const Blas &b, hipStream_t s, int64_t E, Fn fn) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || fork_sides(b, s) != hipSuccess) return MOE_ERR_HIP;
  std::atomic<int> status{MOE_OK};
  std::thread th[kSide];
  for (int i = 0; i < kSide; ++i)
    th[i] = std::thread([&, i] {
      if (hipSetDevice(dev) != hipSuccess) status.store(MOE_ERR_HIP);  // the caller's device
      for (int64_t e = i; e < E && status.load() == MOE_OK; e += kSide) {
        const moe_status st = fn(e, b.side[i], b.ss[i]);
        if (st != MOE_OK) status.store(st);
      }
    });
  for (auto &t : th) t.join();
  if (join_sides(b, s) != hipSuccess) return MOE_ERR_HIP;
  return static_cast<moe_status>(status.load());
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
  Blas *bl = blas();
  if (!bl) return MOE_ERR_HIP;
  rocblas_handle hd = bl->main;
  MOE_TRY_BLAS(rocblas_set_stream(hd, s));
  const float beta = cfg->beta, ib = 1.0f / cfg->beta, bu = cfg->beta_u, ibu = 1.0f / cfg->beta_u;

  int32_t *counts = at<int32_t>(ws, p.counts), *offsets = at<int32_t>(ws, p.offsets);
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
  uint16_t *dgs = at<uint16_t>(ws, p.dgs), *dus = at<uint16_t>(ws, p.dus);
  const uint16_t *Wg = static_cast<const uint16_t *>(w->w_gate);
  const uint16_t *Wu = static_cast<const uint16_t *>(w->w_up);
  const uint16_t *Wd = static_cast<const uint16_t *>(w->w_down);

  // ---- recompute: dispatch, x_lat, the routed experts, y_lat and r -------------------
  MOE_TRY(launch_dispatch(topk_idx, topk_w, bt, k, E, 64, at<uint64_t>(ws, p.masks), counts,
                          offsets, at<int32_t>(ws, p.tile_offsets), perm, inv_perm, w_sorted,
                          s));
  std::vector<int32_t> off_h(E + 1);
  MOE_TRY(hipMemcpyAsync(off_h.data(), offsets, 4 * (E + 1), hipMemcpyDeviceToHost, s));
  MOE_TRY(hipStreamSynchronize(s));
  MOE_TRY_BLAS(gemm_rm(hd, false, true, bt, L, d, x, BF, d, w->w_down_proj, BF, d, 0.0f, xlat,
                       BF, L));
  MOE_TRY(launch_kernel(gather_rows_kernel, grid_for(P * L / 8), dim3(256), 0, s,
                        (const uint16_t *)xlat, (const int32_t *)perm, (int)k, P, L, xg));
  st = for_experts(*bl, s, E, [&](int64_t e, rocblas_handle he, hipStream_t se) -> moe_status {
    (void)se;
    const int64_t q0 = off_h[e], ne = off_h[e + 1] - q0;
    if (ne == 0) return MOE_OK;
    MOE_TRY_BLAS(gemm_rm(he, false, true, ne, I, L, xg + q0 * L, BF, L, Wg + e * I * L, BF, L,
                         0.0f, G + q0 * I, F32, I));
    MOE_TRY_BLAS(gemm_rm(he, false, true, ne, I, L, xg + q0 * L, BF, L, Wu + e * I * L, BF, L,
                         0.0f, U + q0 * I, F32, I));
    return MOE_OK;
  });
  if (st != MOE_OK) return st;
  MOE_TRY(launch_kernel(situ_h_kernel, grid_for(P * I), dim3(256), 0, s, (const float *)G,
                        (const float *)U, (const float *)w_sorted, P, I, beta, ib, bu, ibu, h));
  st = for_experts(*bl, s, E, [&](int64_t e, rocblas_handle he, hipStream_t se) -> moe_status {
    (void)se;
    const int64_t q0 = off_h[e], ne = off_h[e + 1] - q0;
    if (ne == 0) return MOE_OK;
    MOE_TRY_BLAS(gemm_rm(he, false, true, ne, L, I, h + q0 * I, BF, I, Wd + e * L * I, BF, I,
                         0.0f, o + q0 * L, BF, L));
    return MOE_OK;
  });
  if (st != MOE_OK) return st;
  MOE_TRY(launch_kernel(combine_ylat_kernel, dim3((unsigned)bt), dim3(256), 0, s,
                        (const uint16_t *)o, (const int32_t *)inv_perm, (int)k, L,
                        w->latent_gamma, cfg->rms_eps, ylat, rinv, n));
  const uint16_t *shg = static_cast<const uint16_t *>(w->sh_gate);
  const uint16_t *shu = static_cast<const uint16_t *>(w->sh_up);
  const uint16_t *shd = static_cast<const uint16_t *>(w->sh_down);
  if (S > 0) {  // the S shared experts' gate / up rows are one [S I_s][d] matrix each
    MOE_TRY_BLAS(gemm_rm(hd, false, true, bt, SI, d, x, BF, d, shg, BF, d, 0.0f, Gs, F32, SI));
    MOE_TRY_BLAS(gemm_rm(hd, false, true, bt, SI, d, x, BF, d, shu, BF, d, 0.0f, Us, F32, SI));
    MOE_TRY(launch_kernel(situ_h_kernel, grid_for(bt * SI), dim3(256), 0, s, (const float *)Gs,
                          (const float *)Us, (const float *)nullptr, bt, SI, beta, ib, bu, ibu,
                          hs));
  }

  // ---- y = W_up n + sum_s W_ds,s hs_s ----------------------------------------------
  MOE_TRY_BLAS(gemm_rm(hd, true, false, d, L, bt, dy, BF, d, n, BF, L, 0.0f, g->w_up_proj, F32,
                       L));
  MOE_TRY_BLAS(gemm_rm(hd, false, false, bt, L, d, dy, BF, d, w->w_up_proj, BF, L, 0.0f, dn, F32,
                       L));
  for (int64_t sx = 0; sx < S; ++sx) {
    MOE_TRY_BLAS(gemm_rm(hd, true, false, d, Is, bt, dy, BF, d, hs + sx * Is, BF, SI, 0.0f,
                         g->sh_down + sx * d * Is, F32, Is));
    MOE_TRY_BLAS(gemm_rm(hd, false, false, bt, Is, d, dy, BF, d, shd + sx * d * Is, BF, Is, 0.0f,
                         dhs + sx * Is, F32, SI));
  }
  // ---- n = y_lat r gamma ------------------------------------------------------------
  MOE_TRY(colsum(dn, ylat, rinv, bt, L, part, g->latent_gamma, s));
  MOE_TRY(launch_kernel(rms_bwd_kernel, dim3((unsigned)bt), dim3(256), 0, s, (const float *)dn,
                        (const float *)ylat, (const float *)rinv, w->latent_gamma, L, dylat));
  // ---- routed experts ---------------------------------------------------------------
  MOE_TRY(launch_kernel(gather_rows_kernel, grid_for(P * L / 8), dim3(256), 0, s,
                        (const uint16_t *)dylat, (const int32_t *)perm, (int)k, P, L, dyg));
  MOE_TRY(fill_f32(dz, bt * E, s));
  st = for_experts(*bl, s, E, [&](int64_t e, rocblas_handle he, hipStream_t se) -> moe_status {
    (void)se;
    const int64_t q0 = off_h[e], ne = off_h[e + 1] - q0;
    if (ne == 0) {  // no pair chose the expert
      MOE_TRY(fill_f32(g->w_down + e * L * I, L * I, se));
      return MOE_OK;
    }
    MOE_TRY_BLAS(gemm_rm(he, true, false, L, I, ne, dyg + q0 * L, BF, L, h + q0 * I, BF, I, 0.0f,
                         g->w_down + e * L * I, F32, I));
    MOE_TRY_BLAS(gemm_rm(he, false, false, ne, I, L, dyg + q0 * L, BF, L, Wd + e * L * I, BF, I,
                         0.0f, dh + q0 * I, F32, I));
    return MOE_OK;
  });
  if (st != MOE_OK) return st;
  MOE_TRY(launch_kernel(situ_bwd_kernel, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, s, (const float *)dh,
                        (const float *)G, (const float *)U, (const float *)w_sorted,
                        (const int32_t *)perm, topk_idx, (int)k, E, P, I, beta, ib, bu, ibu, dg,
                        du, dz));
  st = for_experts(*bl, s, E, [&](int64_t e, rocblas_handle he, hipStream_t se) -> moe_status {
    (void)se;
    const int64_t q0 = off_h[e], ne = off_h[e + 1] - q0;
    if (ne == 0) {
      MOE_TRY(fill_f32(g->w_gate + e * I * L, I * L, se));
      MOE_TRY(fill_f32(g->w_up + e * I * L, I * L, se));
      return MOE_OK;
    }
    MOE_TRY_BLAS(gemm_rm(he, true, false, I, L, ne, dg + q0 * I, BF, I, xg + q0 * L, BF, L, 0.0f,
                         g->w_gate + e * I * L, F32, L));
    MOE_TRY_BLAS(gemm_rm(he, true, false, I, L, ne, du + q0 * I, BF, I, xg + q0 * L, BF, L, 0.0f,
                         g->w_up + e * I * L, F32, L));
    MOE_TRY_BLAS(gemm_rm(he, false, false, ne, L, I, dg + q0 * I, BF, I, Wg + e * I * L, BF, L,
                         0.0f, dxg + q0 * L, F32, L));
    MOE_TRY_BLAS(gemm_rm(he, false, false, ne, L, I, du + q0 * I, BF, I, Wu + e * I * L, BF, L,
                         1.0f, dxg + q0 * L, F32, L));
    return MOE_OK;
  });
  if (st != MOE_OK) return st;
  MOE_TRY(launch_kernel(combine_rows_kernel, grid_for(bt * L), dim3(256), 0, s,
                        (const float *)dxg, (const int32_t *)inv_perm, (int)k, bt, L, dxlat));
  // ---- x_lat = W_down_proj x, and the router ------------------------------------------
  MOE_TRY_BLAS(gemm_rm(hd, true, false, L, d, bt, dxlat, BF, L, x, BF, d, 0.0f, g->w_down_proj,
                       F32, d));
  MOE_TRY_BLAS(gemm_rm(hd, false, false, bt, d, L, dxlat, BF, L, w->w_down_proj, BF, d, 0.0f,
                       g->dx, F32, d));
  MOE_TRY(launch_kernel(cvt_bf16_kernel, grid_for(bt * E), dim3(256), 0, s, (const float *)dz,
                        bt * E, dz16));
  MOE_TRY_BLAS(gemm_rm(hd, true, false, E, d, bt, dz16, BF, E, x, BF, d, 0.0f, g->w_router, F32,
                       d));
  MOE_TRY_BLAS(gemm_rm(hd, false, false, bt, d, E, dz16, BF, E, w->w_router, BF, d, 1.0f, g->dx,
                       F32, d));
  MOE_TRY(colsum(dz, nullptr, nullptr, bt, E, part, g->router_bias, s));
  // ---- shared experts ---------------------------------------------------------------
  if (S > 0) {
    MOE_TRY(launch_kernel(situ_bwd_kernel, dim3((unsigned)((bt + 3) / 4)), dim3(256), 0, s, (const float *)dhs,
                          (const float *)Gs, (const float *)Us, (const float *)nullptr,
                          (const int32_t *)nullptr, (const int32_t *)nullptr, 1, E, bt, SI, beta,
                          ib, bu, ibu, dgs, dus, (float *)nullptr));
    MOE_TRY_BLAS(gemm_rm(hd, true, false, SI, d, bt, dgs, BF, SI, x, BF, d, 0.0f, g->sh_gate, F32,
                         d));
    MOE_TRY_BLAS(gemm_rm(hd, true, false, SI, d, bt, dus, BF, SI, x, BF, d, 0.0f, g->sh_up, F32,
                         d));
    MOE_TRY_BLAS(gemm_rm(hd, false, false, bt, d, SI, dgs, BF, SI, shg, BF, d, 1.0f, g->dx, F32,
                         d));
    MOE_TRY_BLAS(gemm_rm(hd, false, false, bt, d, SI, dus, BF, SI, shu, BF, d, 1.0f, g->dx, F32,
                         d));
  }
  return MOE_OK;
}
