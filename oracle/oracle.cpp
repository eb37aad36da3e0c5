// oracle.cpp -- plain fp64 CPU oracle of the Stable LatentMoE layer forward.
//
// TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke
// check and the benchmark's CPU-baseline leg, never by the product path.
// Written directly from the layer's definition; shares no code with the GPU
// library.  Every dot product runs in fp64 in index order.
#include "oracle.h"

#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

namespace {

const int32_t ORC_F64 = 64;  // internal: fully decoded fp64 copy

int64_t elem_bytes(int32_t dt) {
  switch (dt) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_FP8E4M3: return 1;
    case ORC_MXFP4: return 1;  // (half a byte per element)
    case ORC_MXFP8: return 1;
    case ORC_F64: return 8;
  }
  return 0;
}

bool valid_mat(const orc_mat *m) {
  if (!m || !m->data || m->rows <= 0 || m->cols <= 0 || m->n_mats <= 0) return false;
  if (elem_bytes(m->dtype) == 0) return false;
  if (m->dtype == ORC_FP8E4M3 && (!m->scale || m->rows % 128 || m->cols % 128)) return false;
  if ((m->dtype == ORC_MXFP4 || m->dtype == ORC_MXFP8) && (!m->scale || m->cols % 32))
    return false;
  return true;
}

// Decode row r of matrix `mat` into buf[cols] (exact).
void decode_row(const orc_mat *m, int64_t mat, int64_t r, double *buf) {
  const int64_t cols = m->cols;
  const int64_t base = (mat * m->rows + r) * cols;
  switch (m->dtype) {
    case ORC_F32: {
      const float *p = static_cast<const float *>(m->data) + base;
      for (int64_t c = 0; c < cols; ++c) buf[c] = (double)p[c];
      break;
    }
    case ORC_BF16: {
      const uint16_t *p = static_cast<const uint16_t *>(m->data) + base;
      for (int64_t c = 0; c < cols; ++c) buf[c] = orc_bf16_to_double(p[c]);
      break;
    }
    case ORC_FP8E4M3: {
      const uint8_t *p = static_cast<const uint8_t *>(m->data) + base;
      const int64_t bc = cols / 128;
      const float *srow = static_cast<const float *>(m->scale) + (mat * (m->rows / 128) + r / 128) * bc;
      for (int64_t c = 0; c < cols; ++c)
        buf[c] = orc_e4m3_to_double(p[c]) * (double)srow[c / 128];
      break;
    }
    case ORC_MXFP4: {
      // element c: nibble (c odd ? high : low) of byte c/2 of the row, times
      // the E8M0 scale of its 32-element block
      const uint8_t *p = static_cast<const uint8_t *>(m->data) + base / 2;
      const uint8_t *srow = static_cast<const uint8_t *>(m->scale) + (mat * m->rows + r) * (cols / 32);
      for (int64_t c = 0; c < cols; ++c) {
        const uint8_t code = (c & 1) ? (uint8_t)(p[c / 2] >> 4) : (uint8_t)(p[c / 2] & 0xF);
        buf[c] = orc_e2m1_to_double(code) * orc_e8m0_to_double(srow[c / 32]);
      }
      break;
    }
    case ORC_MXFP8: {
      // element c: e4m3 code c of the row times the E8M0 scale of its block
      const uint8_t *p = static_cast<const uint8_t *>(m->data) + base;
      const uint8_t *srow = static_cast<const uint8_t *>(m->scale) + (mat * m->rows + r) * (cols / 32);
      for (int64_t c = 0; c < cols; ++c)
        buf[c] = orc_e4m3_to_double(p[c]) * orc_e8m0_to_double(srow[c / 32]);
      break;
    }
    case ORC_F64: {
      const double *p = static_cast<const double *>(m->data) + base;
      std::memcpy(buf, p, sizeof(double) * cols);
      break;
    }
  }
}

// A fully decoded fp64 copy of every matrix of m.
struct Decoded {
  std::vector<double> data;
  orc_mat mat;
  explicit Decoded(const orc_mat *m) {
    data.resize((size_t)(m->n_mats * m->rows * m->cols));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m->n_mats * m->rows; ++i)
      decode_row(m, i / m->rows, i % m->rows, data.data() + i * m->cols);
    mat = *m;
    mat.data = data.data();
    mat.dtype = ORC_F64;
    mat.scale = nullptr;
  }
};

double dot(const double *a, const double *b, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

}  // namespace

extern "C" {

void orc_set_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }
int orc_get_threads(void) { return omp_get_max_threads(); }

double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// OCP fp8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
// infinities; S.1111.111 is NaN; exponent field 0 encodes subnormals m * 2^-9.
double orc_e4m3_to_double(uint8_t code) {
  const int sign = code >> 7;
  const int ex = (code >> 3) & 0xF;
  const int man = code & 0x7;
  double v;
  if (ex == 0xF && man == 0x7) v = std::nan("");
  else if (ex == 0) v = std::ldexp((double)man, -9);
  else v = std::ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

// OCP MX FP4 E2M1: exponent field 0 is subnormal (m * 2^-1), else
// (1 + m/2) * 2^(e - 1); the largest magnitude is 6.
double orc_e2m1_to_double(uint8_t code) {
  const int sign = (code >> 3) & 1;
  const int ex = (code >> 1) & 0x3;
  const int man = code & 0x1;
  const double v = ex == 0 ? 0.5 * man : std::ldexp(1.0 + man / 2.0, ex - 1);
  return sign ? -v : v;
}

// OCP MX E8M0 scale: an unsigned biased exponent, 2^(code - 127); 0xFF is NaN.
double orc_e8m0_to_double(uint8_t code) {
  if (code == 0xFF) return std::nan("");
  return std::ldexp(1.0, (int)code - 127);
}

// Nearest E4M3 value: |v| = 2^e (1 + f), the mantissa rounded to 3 bits
// (normal, e >= -6) or |v| rounded to a multiple of 2^-9 (subnormal), ties to
// even, at most 448.
uint8_t orc_double_to_e4m3(double v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  const double a = std::fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);  // a = m 2^e2, m in [0.5, 1)
  const int e = e2 - 1;  // a in [2^e, 2^(e+1))
  if (e < -6) {
    const double q = std::nearbyint(std::ldexp(a, 9));  // multiples of 2^-9, ties to even
    return sign | (uint8_t)q;  // q == 8 is the smallest normal, code 0x08
  }
  double mant = std::nearbyint((std::ldexp(a, -e) - 1.0) * 8.0);
  int eb = e + 7;
  if (mant == 8.0) {
    mant = 0.0;
    eb += 1;
  }
  const int code = (eb << 3) | (int)mant;
  return sign | (uint8_t)(code > 0x7E ? 0x7E : code);
}

double orc_round_bf16(double v) {
  if (v == 0.0 || !std::isfinite(v)) return v;
  int e2;
  std::frexp(v, &e2);                          // |v| in [2^(e2-1), 2^e2)
  const int q = std::max(e2 - 1 - 7, -133);    // weight of the last bf16 bit
  return std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);  // exact scaling; RNE
}

int orc_mx8_quantize(const double *x, int64_t n, int64_t block, uint8_t *codes,
                     uint8_t *scales) {
  if (!x || !codes || !scales || block <= 0 || n % block) return -1;
  for (int64_t b0 = 0; b0 < n; b0 += block) {
    double amax = 0.0;
    for (int64_t i = 0; i < block; ++i) amax = std::max(amax, std::fabs(x[b0 + i]));
    int shared = -127;
    if (amax > 0.0) {
      int e2;
      std::frexp(amax, &e2);
      shared = std::min(127, std::max(-127, (e2 - 1) - 8));
    }
    scales[b0 / block] = (uint8_t)(shared + 127);
    for (int64_t i = 0; i < block; ++i)
      codes[b0 + i] = orc_double_to_e4m3(std::ldexp(x[b0 + i], -shared));
  }
  return 0;
}

// x replaced by its MX FP8 quantisation (dequantised exactly), blocks of
// `block`, the codes decided on x rounded to bf16 (on_bf16) or on x itself.
static void mx8_round_trip(double *x, int64_t n, int64_t block, bool on_bf16) {
  std::vector<uint8_t> codes((size_t)n), scales((size_t)(n / block));
  if (on_bf16)
    for (int64_t i = 0; i < n; ++i) x[i] = orc_round_bf16(x[i]);
  orc_mx8_quantize(x, n, block, codes.data(), scales.data());
  for (int64_t i = 0; i < n; ++i)
    x[i] = orc_e4m3_to_double(codes[i]) * orc_e8m0_to_double(scales[i / block]);
}

double orc_decode(const orc_mat *m, int64_t mat, int64_t r, int64_t c) {
  std::vector<double> row((size_t)m->cols);
  decode_row(m, mat, r, row.data());
  return row[(size_t)c];
}

void orc_matvec(const orc_mat *m, int64_t mat, const double *in, double *out) {
  if (m->dtype == ORC_F64) {
    const double *base = static_cast<const double *>(m->data) + mat * m->rows * m->cols;
#pragma omp parallel for schedule(static) if (!omp_in_parallel() && m->rows >= 64)
    for (int64_t r = 0; r < m->rows; ++r) out[r] = dot(base + r * m->cols, in, m->cols);
    return;
  }
#pragma omp parallel if (!omp_in_parallel() && m->rows >= 64)
  {
    std::vector<double> row((size_t)m->cols);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < m->rows; ++r) {
      decode_row(m, mat, r, row.data());
      out[r] = dot(row.data(), in, m->cols);
    }
  }
}

double orc_sigmoid(double z) { return 1.0 / (1.0 + std::exp(-z)); }

// SiTU gate: Swish with its unbounded factor replaced by beta*tanh(g/beta).
double orc_phi(double g, double beta) { return orc_sigmoid(g) * beta * std::tanh(g / beta); }

// SiTU up-branch bound: beta_u * tanh(u / beta_u).
double orc_psi(double u, double beta_u) { return beta_u * std::tanh(u / beta_u); }

int orc_router_logits(const orc_shape *s, const orc_weights *w, const orc_mat *x,
                      const int64_t *rows, int64_t n_rows, double *z_out) {
  if (!s || !w || !valid_mat(x) || !valid_mat(&w->w_router) || !z_out || n_rows < 0) return -1;
  const int64_t E = s->n_experts, d = s->d;
  if (w->w_router.rows != E || w->w_router.cols != d || x->cols != d) return -1;
  Decoded wr(&w->w_router);
#pragma omp parallel
  {
    std::vector<double> xr((size_t)d);
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < n_rows; ++i) {
      const int64_t t = rows ? rows[i] : i;
      decode_row(x, 0, t, xr.data());
      for (int64_t e = 0; e < E; ++e) {
        double acc = dot(static_cast<const double *>(wr.mat.data) + e * d, xr.data(), d);
        if (w->router_bias) acc += (double)w->router_bias[e];
        z_out[i * E + e] = acc;
      }
    }
  }
  return 0;
}

int orc_quantile(const float *z32, int64_t bt, int64_t n_experts, int64_t m, float *zeta) {
  if (!z32 || !zeta || bt <= 0 || n_experts <= 0 || m < 1 || m > bt) return -1;
#pragma omp parallel
  {
    std::vector<float> col((size_t)bt);
#pragma omp for schedule(static)
    for (int64_t e = 0; e < n_experts; ++e) {
      for (int64_t t = 0; t < bt; ++t) col[t] = z32[t * n_experts + e];
      std::sort(col.begin(), col.end(), [](float a, float b) { return a > b; });
      zeta[e] = col[m - 1];
    }
  }
  return 0;
}

int orc_topk(const float *z32, const float *alpha, const double *z64, int64_t bt,
             int64_t n_experts, int64_t k, int32_t *idx, double *w) {
  if (!z32 || !idx || !w || bt < 0 || n_experts <= 0 || k < 1 || k > n_experts) return -1;
#pragma omp parallel
  {
    std::vector<std::pair<float, int32_t>> cand((size_t)n_experts);
    std::vector<int32_t> pick((size_t)k);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < bt; ++t) {
      for (int64_t e = 0; e < n_experts; ++e) {
        // the cutoff-adjusted logit, subtracted in fp32
        const float r = z32[t * n_experts + e] - (alpha ? alpha[e] : 0.0f);
        cand[e] = {r, (int32_t)e};
      }
      std::sort(cand.begin(), cand.end(),
                [](const std::pair<float, int32_t> &a, const std::pair<float, int32_t> &b) {
                  if (a.first != b.first) return a.first > b.first;
                  return a.second < b.second;
                });
      for (int64_t j = 0; j < k; ++j) pick[j] = cand[j].second;
      std::sort(pick.begin(), pick.end());
      for (int64_t j = 0; j < k; ++j) {
        const int32_t e = pick[j];
        idx[t * k + j] = e;
        const double z = z64 ? z64[t * n_experts + e] : (double)z32[t * n_experts + e];
        w[t * k + j] = orc_sigmoid(z);
      }
    }
  }
  return 0;
}

int orc_dispatch(const int32_t *idx, int64_t bt, int64_t k, int64_t n_experts,
                 int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm) {
  if (!idx || !counts || !offsets || !perm || !inv_perm || bt < 0 || k < 1) return -1;
  for (int64_t e = 0; e < n_experts; ++e) counts[e] = 0;
  for (int64_t p = 0; p < bt * k; ++p) {
    const int32_t e = idx[p];
    if (e < 0 || e >= n_experts) return -1;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill((size_t)n_experts, 0);
  // tokens in ascending order: each expert's segment lists its tokens ascending
  for (int64_t t = 0; t < bt; ++t)
    for (int64_t j = 0; j < k; ++j) {
      const int64_t p = t * k + j;
      const int32_t e = idx[p];
      const int32_t pos = offsets[e] + fill[e]++;
      perm[pos] = (int32_t)p;
      inv_perm[p] = pos;
    }
  return 0;
}

int orc_expert(const orc_shape *s, const orc_mat *w_gate, const orc_mat *w_up,
               const orc_mat *w_down, int64_t mat, const double *x_lat, double *o) {
  if (!s || !w_gate || !w_up || !w_down || !x_lat || !o) return -1;
  const int64_t I = s->expert_inter, L = s->latent, qb = s->act_mx_block;
  if (qb < 0 || (qb > 0 && (L % qb || I % qb))) return -1;
  std::vector<double> xin(x_lat, x_lat + L);
  const bool on_bf16 = s->act_mx_exact == 0;
  if (qb > 0) mx8_round_trip(xin.data(), L, qb, on_bf16);  // gate/up read MX FP8 x_lat
  std::vector<double> g((size_t)I), u((size_t)I), h((size_t)I);
  orc_matvec(w_gate, mat, xin.data(), g.data());
  orc_matvec(w_up, mat, xin.data(), u.data());
  for (int64_t i = 0; i < I; ++i) h[i] = orc_phi(g[i], s->beta) * orc_psi(u[i], s->beta_u);
  if (qb > 0) mx8_round_trip(h.data(), I, qb, on_bf16);  // and the down GEMM MX FP8 h
  orc_matvec(w_down, mat, h.data(), o);
  return 0;
}

// RMSNorm of one row: out = x / sqrt(mean(x^2) + eps) * gamma (gamma NULL = 1).
void orc_rmsnorm(const double *x, int64_t n, const float *gamma, double eps, double *out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / std::sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = x[i] * inv * (gamma ? (double)gamma[i] : 1.0);
}

// Dense FFN of one row: the SiTU-GLU of the experts at width d and
// intermediate width I, on the RMS-normalised row, added to r.
int orc_dense_ffn(const orc_shape *s, const orc_mat *w_gate, const orc_mat *w_up,
                  const orc_mat *w_down, const float *gamma, const double *x, const double *r,
                  double *y) {
  if (!s || !w_gate || !w_up || !w_down || !x || !y || s->d <= 0 || s->expert_inter <= 0)
    return -1;
  if (w_gate->rows != s->expert_inter || w_gate->cols != s->d || w_up->rows != s->expert_inter ||
      w_up->cols != s->d || w_down->rows != s->d || w_down->cols != s->expert_inter)
    return -1;
  const int64_t d = s->d;
  std::vector<double> n((size_t)d), o((size_t)d);
  orc_rmsnorm(x, d, gamma, s->rms_eps, n.data());
  orc_shape e = *s;
  e.latent = d;  // the expert GLU reads its input at width "latent"
  if (orc_expert(&e, w_gate, w_up, w_down, 0, n.data(), o.data())) return -1;
  for (int64_t i = 0; i < d; ++i) y[i] = (r ? r[i] : 0.0) + o[i];
  return 0;
}

int orc_combine_norm(const orc_shape *s, const double *o, const double *w,
                     const float *gamma, double *y_lat, double *n) {
  if (!s || !o || !w || !y_lat || !n) return -1;
  const int64_t L = s->latent, k = s->top_k;
  for (int64_t l = 0; l < L; ++l) {
    double acc = 0.0;
    for (int64_t j = 0; j < k; ++j) acc += w[j] * o[j * L + l];
    y_lat[l] = acc;
  }
  double ss = 0.0;
  for (int64_t l = 0; l < L; ++l) ss += y_lat[l] * y_lat[l];
  const double inv = 1.0 / std::sqrt(ss / (double)L + s->rms_eps);
  for (int64_t l = 0; l < L; ++l) n[l] = y_lat[l] * inv * (gamma ? (double)gamma[l] : 1.0);
  return 0;
}

int orc_shared(const orc_shape *s, const orc_weights *w, const double *x_t, double *out) {
  if (!s || !w || !x_t || !out) return -1;
  const int64_t d = s->d, Is = s->shared_inter;
  std::vector<double> g((size_t)Is), u((size_t)Is), h((size_t)Is), part((size_t)d);
  for (int64_t r = 0; r < d; ++r) out[r] = 0.0;
  for (int64_t j = 0; j < s->n_shared; ++j) {
    orc_matvec(&w->sh_gate, j, x_t, g.data());
    orc_matvec(&w->sh_up, j, x_t, u.data());
    for (int64_t i = 0; i < Is; ++i) h[i] = orc_phi(g[i], s->beta) * orc_psi(u[i], s->beta_u);
    orc_matvec(&w->sh_down, j, h.data(), part.data());
    for (int64_t r = 0; r < d; ++r) out[r] += part[r];
  }
  return 0;
}

int orc_output(const orc_shape *s, const orc_weights *w, const double *n, const double *x_t,
               double *y) {
  if (!s || !w || !n || !x_t || !y) return -1;
  const int64_t d = s->d;
  std::vector<double> up((size_t)d), sh((size_t)d);
  orc_matvec(&w->w_up_proj, 0, n, up.data());
  orc_shared(s, w, x_t, sh.data());
  for (int64_t r = 0; r < d; ++r) y[r] = up[r] + sh[r];
  return 0;
}

int orc_forward(const orc_shape *s, const orc_weights *w, const orc_mat *x, int64_t bt,
                int32_t cutoff_mode, const float *alpha_given, float *z32_out,
                float *zeta_out, int32_t *idx_out, double *wts_out, int32_t *counts,
                int32_t *offsets, int32_t *perm, int32_t *inv_perm, double *y) {
  if (!s || !w || !x || !y || bt <= 0) return -1;
  const int64_t E = s->n_experts, k = s->top_k, d = s->d, L = s->latent, P = bt * k;
  if (k < 1 || k > E) return -1;
  if (cutoff_mode != ORC_CUTOFF_GIVEN && cutoff_mode != ORC_CUTOFF_BATCH) return -1;

  // 1. router logits, fp64, and their fp32 rounding
  std::vector<double> z64((size_t)(bt * E));
  if (orc_router_logits(s, w, x, nullptr, bt, z64.data()) != 0) return -1;
  std::vector<float> z32((size_t)(bt * E));
  for (int64_t i = 0; i < bt * E; ++i) z32[i] = (float)z64[i];

  // 2. cutoffs
  std::vector<float> alpha((size_t)E, 0.0f);
  if (cutoff_mode == ORC_CUTOFF_BATCH) {
    int64_t m = (bt * k + E - 1) / E;
    m = std::max<int64_t>(1, std::min<int64_t>(m, bt));
    orc_quantile(z32.data(), bt, E, m, alpha.data());
  } else if (alpha_given) {
    for (int64_t e = 0; e < E; ++e) alpha[e] = alpha_given[e];
  }

  // 3. top-k
  std::vector<int32_t> idx((size_t)P);
  std::vector<double> wts((size_t)P);
  orc_topk(z32.data(), alpha.data(), z64.data(), bt, E, k, idx.data(), wts.data());

  // 4. dispatch
  std::vector<int32_t> cnt((size_t)E), off((size_t)(E + 1)), pm((size_t)P), ipm((size_t)P);
  if (orc_dispatch(idx.data(), bt, k, E, cnt.data(), off.data(), pm.data(), ipm.data()) != 0)
    return -1;

  // decoded fp64 copies of the weights, so the per-token loops stay plain
  Decoded wdp(&w->w_down_proj), wg(&w->w_gate), wu(&w->w_up), wd(&w->w_down),
      wup(&w->w_up_proj), sg(&w->sh_gate), su(&w->sh_up), sd(&w->sh_down);
  orc_weights wdec = *w;
  wdec.w_down_proj = wdp.mat; wdec.w_gate = wg.mat; wdec.w_up = wu.mat;
  wdec.w_down = wd.mat; wdec.w_up_proj = wup.mat;
  wdec.sh_gate = sg.mat; wdec.sh_up = su.mat; wdec.sh_down = sd.mat;

  // 5. x_lat = W_down_proj x
  std::vector<double> xd((size_t)(bt * d)), xlat((size_t)(bt * L));
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < bt; ++t) {
    decode_row(x, 0, t, xd.data() + t * d);
    orc_matvec(&wdec.w_down_proj, 0, xd.data() + t * d, xlat.data() + t * L);
  }

  // 6. expert outputs per pair, slot order
  std::vector<double> o((size_t)(P * L));
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < P; ++p) {
    const int64_t t = p / k;
    orc_expert(s, &wdec.w_gate, &wdec.w_up, &wdec.w_down, idx[p], xlat.data() + t * L,
               o.data() + p * L);
  }

  // 7-8. combine + latent RMSNorm, then W_up_proj plus the shared experts
#pragma omp parallel
  {
    std::vector<double> ylat((size_t)L), nrm((size_t)L);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < bt; ++t) {
      orc_combine_norm(s, o.data() + t * k * L, wts.data() + t * k, w->gamma, ylat.data(),
                       nrm.data());
      orc_output(s, &wdec, nrm.data(), xd.data() + t * d, y + t * d);
    }
  }

  if (z32_out) std::memcpy(z32_out, z32.data(), sizeof(float) * bt * E);
  if (zeta_out) std::memcpy(zeta_out, alpha.data(), sizeof(float) * E);
  if (idx_out) std::memcpy(idx_out, idx.data(), sizeof(int32_t) * P);
  if (wts_out) std::memcpy(wts_out, wts.data(), sizeof(double) * P);
  if (counts) std::memcpy(counts, cnt.data(), sizeof(int32_t) * E);
  if (offsets) std::memcpy(offsets, off.data(), sizeof(int32_t) * (E + 1));
  if (perm) std::memcpy(perm, pm.data(), sizeof(int32_t) * P);
  if (inv_perm) std::memcpy(inv_perm, ipm.data(), sizeof(int32_t) * P);
  return 0;
}

}  // extern "C"
