/*
 * oracle.h -- plain, slow fp64 CPU oracle of the Stable LatentMoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code with the GPU library.
 *
 * What it computes (the plain definition of the layer):
 *   Kimi K3 Stable LatentMoE as described on tech.news18a.com
 *   "KimiK3的StableLatentMoE架构解析" (module structure, figure 1; forward flow,
 *   figure 2; the three stability techniques: SiTU-GLU, RMSNorm before up,
 *   Quantile Balancing) and on mkdocs.reaper.mx "Vue d'ensemble de
 *   l'architecture" (per-token path, steps c-g; parameter budget table).
 *
 *   1. logits z[t][e] = sum_i x[t][i] W_r[e][i] + b[e];  scores s = sigmoid(z)
 *   2. cutoff (BATCH mode): zeta[e] = m-th largest of column e of fp32 z,
 *      m = clamp(ceil(bt*k/E), 1, bt); GIVEN mode uses a caller's alpha.
 *   3. r = fp32(z) - alpha in fp32; per token the k experts of largest r
 *      (equal r: lower expert id first), listed in ascending expert id;
 *      combine weight w = s at the chosen expert (not renormalised).
 *   4. dispatch: per-expert counts, exclusive offsets, pairs p = t*k + j
 *      ordered by (expert asc, token asc), and the inverse permutation.
 *   5. x_lat = W_down_proj x                                     (d -> L)
 *   6. per pair: o = W_d,e (phi(W_g,e x_lat) * psi(W_u,e x_lat))  (width L)
 *   7. y_lat = sum_j w_j o_j (j ascending);  n = y_lat / sqrt(mean(y_lat^2) + eps) * gamma
 *   8. y = W_up_proj n + sum_{j < S} W_ds,j (phi(W_gs,j x) * psi(W_us,j x))
 *   phi(g) = sigmoid(g) * beta * tanh(g / beta),  psi(u) = beta_u * tanh(u / beta_u)
 *
 * Every dot product is accumulated in fp64 in index order.  Inputs are
 * decoded exactly: fp32 and bf16 widen, an fp8 e4m3fn code times its fp32
 * 128x128 block scale is exact in fp64, and so is an MXFP4 E2M1 code times
 * its power-of-two E8M0 block scale.
 *
 * Parity pins (tests/test_oracle_pins.py): closed forms, invariants and
 * brute force as listed there; step 8 (orc_output) by exact dyadic closed
 * forms at the SiTU caps, where phi * psi is exactly beta * beta_u.  The
 * layer output as a whole is pinned only through those properties: the
 * pages print no worked numeric example of it.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8E4M3 = 2, ORC_MXFP4 = 3, ORC_MXFP8 = 4 };
enum { ORC_CUTOFF_GIVEN = 0, ORC_CUTOFF_BATCH = 1 };

/* n_mats matrices of rows x cols, row-major, raw storage.
 *   ORC_FP8E4M3: one byte per element; scale -> float [n_mats][rows/128][cols/128],
 *                one factor per 128 x 128 block.
 *   ORC_MXFP4:   OCP MX FP4 -- two E2M1 codes per byte, element 2i of a row in
 *                the low nibble of byte i, 2i+1 in the high nibble (a row is
 *                cols/2 bytes); scale -> uint8 E8M0 codes [n_mats][rows][cols/32],
 *                one per 32 consecutive elements of a row.
 *   ORC_MXFP8:   OCP MX FP8 -- one e4m3fn code per byte; scale as for ORC_MXFP4.
 * (OCP Microscaling Formats (MX) Specification v1.0: element types FP4 E2M1 and
 * FP8 E4M3, scale type E8M0, block size 32.) */
typedef struct {
  const void *data;
  int32_t dtype;
  const void *scale;
  int64_t n_mats, rows, cols;
} orc_mat;

typedef struct {
  int64_t d, latent, n_experts, top_k, expert_inter, n_shared, shared_inter;
  double beta, beta_u, rms_eps;
  /* 0: the routed experts read their inputs exactly.  32: each expert GEMM
   * reads its input (x_lat for gate/up, h for down) quantised to OCP MX FP8
   * E4M3 with one E8M0 scale per 32 consecutive elements (orc_mx8_quantize),
   * and the routing weight multiplies the expert output as always.  Where
   * floating point decides a code, the decision is taken in the precision of
   * the stored input: by default the input rounded to bf16 (orc_round_bf16),
   * the precision in which the layer holds x_lat and h when it quantises
   * them (the pages fix none).  act_mx_exact = 1 decides the codes on the
   * exact fp64 input instead, the plain reading of the MX conversion. */
  int64_t act_mx_block;
  int64_t act_mx_exact;
} orc_shape;

typedef struct {
  orc_mat w_router;                 /* [1][E][d] */
  const float *router_bias;         /* [E] or NULL */
  orc_mat w_down_proj;              /* [1][L][d] */
  orc_mat w_gate, w_up;             /* [E][I][L] */
  orc_mat w_down;                   /* [E][L][I] */
  const float *gamma;               /* [L] */
  orc_mat w_up_proj;                /* [1][d][L] */
  orc_mat sh_gate, sh_up;           /* [S][I_s][d] */
  orc_mat sh_down;                  /* [S][d][I_s] */
} orc_weights;

/* OpenMP threads of the oracle's parallel loops (n >= 1), and the current
 * count: the CPU baseline is timed at the host's core count and at one core. */
void orc_set_threads(int n);
int orc_get_threads(void);

/* One element, decoded exactly. */
double orc_decode(const orc_mat *m, int64_t mat, int64_t r, int64_t c);
double orc_bf16_to_double(uint16_t bits);
double orc_e4m3_to_double(uint8_t code);
/* OCP MX element FP4 E2M1 (low 4 bits of code): sign, 2 exponent bits with
 * bias 1, 1 mantissa bit; no infinities or NaN.  E8M0 scale: 2^(code - 127),
 * code 255 is NaN. */
double orc_e2m1_to_double(uint8_t code);
double orc_e8m0_to_double(uint8_t code);

/* OCP MX FP8 (E4M3) quantisation of x[n] in blocks of `block` consecutive
 * elements (OCP Microscaling Formats (MX) Specification v1.0, the conversion
 * of a vector of scalars to an MX block): per block the shared exponent is
 * floor(log2(max |x|)) - 8 (8 = the largest E4M3 exponent), clamped to
 * [-127, 127] (-127 for an all-zero block); each element is x / 2^shared
 * rounded to the nearest E4M3 value, ties to even, magnitudes beyond 448
 * saturating to 448.  codes[n] E4M3 bytes, scales[n / block] E8M0 codes
 * (shared + 127).  n a multiple of block. */
int orc_mx8_quantize(const double *x, int64_t n, int64_t block, uint8_t *codes, uint8_t *scales);
/* Nearest E4M3 code of a double (ties to even, saturating at +-448). */
uint8_t orc_double_to_e4m3(double v);
/* Nearest bf16 value of a finite double within the bf16 range (8 significant
 * bits, ties to even; below 2^-126 multiples of 2^-133). */
double orc_round_bf16(double v);

/* out[r] = sum_c M[mat][r][c] in[c], fp64, c ascending. */
void orc_matvec(const orc_mat *m, int64_t mat, const double *in, double *out);

double orc_sigmoid(double z);
double orc_phi(double g, double beta);
double orc_psi(double u, double beta_u);

/* Step 1 for the token rows listed (rows == NULL: rows 0..n_rows-1).
 * x is [bt][d] raw storage.  z_out [n_rows][E] fp64. */
int orc_router_logits(const orc_shape *s, const orc_weights *w, const orc_mat *x,
                      const int64_t *rows, int64_t n_rows, double *z_out);

/* Step 2: zeta[e] = m-th largest of z32[.][e] over bt tokens. */
int orc_quantile(const float *z32, int64_t bt, int64_t n_experts, int64_t m, float *zeta);

/* Step 3.  z32 [bt][E] fp32 logits, alpha [E] (NULL: 0), z64 [bt][E] fp64 logits
 * for the combine weights (NULL: the fp32 logits are used).  idx [bt][k]
 * ascending expert ids, w [bt][k]. */
int orc_topk(const float *z32, const float *alpha, const double *z64, int64_t bt,
             int64_t n_experts, int64_t k, int32_t *idx, double *w);

/* Step 4. offsets has E+1 entries. */
int orc_dispatch(const int32_t *idx, int64_t bt, int64_t k, int64_t n_experts,
                 int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm);

/* Step 6 for one pair: o = W_d[e] (phi(W_g[e] xl) * psi(W_u[e] xl)).  The
 * three orc_mat may hold all experts (mat = e) or just one (mat = 0). */
int orc_expert(const orc_shape *s, const orc_mat *w_gate, const orc_mat *w_up,
               const orc_mat *w_down, int64_t mat, const double *x_lat, double *o);

/* Step 7 for one token: o [k][L] expert outputs in slot order, w [k]. */
int orc_combine_norm(const orc_shape *s, const double *o, const double *w,
                     const float *gamma, double *y_lat, double *n);

/* Shared experts on one token: out [d] = sum_j W_ds,j (phi(W_gs,j x) psi(W_us,j x)). */
int orc_shared(const orc_shape *s, const orc_weights *w, const double *x_t, double *out);

/* Step 8 for one token: y = W_up_proj n + shared(x). */
int orc_output(const orc_shape *s, const orc_weights *w, const double *n,
               const double *x_t, double *y);

/* The whole layer on bt tokens (small shapes).  Outputs may be NULL except y.
 * alpha_given: GIVEN-mode cutoffs (NULL: 0).  z32 [bt][E], zeta [E] (BATCH),
 * idx [bt][k], wts [bt][k], counts [E], offsets [E+1], perm/inv_perm [bt*k],
 * y [bt][d] fp64. */
/* ---- Dense layer-1 FFN (a second workload of the same building blocks) ----
 * mkdocs.reaper.mx "Vue d'ensemble de l'architecture": section "Le décompte des
 * couches" (layer 1 is dense: a full-width SiTU-GLU FFN of intermediate width
 * 33 792, no routing) and section "Ce que fait une couche" (each sublayer is
 * preceded by an RMSNorm, and its output is summed into the block
 * representation).  For one token row x[d]:
 *   n = x / sqrt(mean(x^2) + eps) * gamma
 *   y = r + W_d (phi(W_g n) * psi(W_u n))
 * with s->d the width, s->expert_inter the intermediate width I and
 * s->beta, s->beta_u, s->rms_eps; w_gate, w_up hold [1][I][d], w_down [1][d][I];
 * gamma [d] or NULL (= 1); r [d] or NULL (= 0). */
void orc_rmsnorm(const double *x, int64_t n, const float *gamma, double eps, double *out);
int orc_dense_ffn(const orc_shape *s, const orc_mat *w_gate, const orc_mat *w_up,
                  const orc_mat *w_down, const float *gamma, const double *x, const double *r,
                  double *y);

int orc_forward(const orc_shape *s, const orc_weights *w, const orc_mat *x, int64_t bt,
                int32_t cutoff_mode, const float *alpha_given, float *z32_out,
                float *zeta_out, int32_t *idx_out, double *wts_out, int32_t *counts,
                int32_t *offsets, int32_t *perm, int32_t *inv_perm, double *y);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
