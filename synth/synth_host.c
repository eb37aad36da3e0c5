/*
 * synth_host.c -- host (CPU) generator of seeded synthetic layer inputs.
 *
 * Builds with gcc into libsynth_host.so.  Produces the same bits as the
 * device generator in synth_dev.hip (both expand synth_rng.h).  Holds no
 * arithmetic of the MoE layer.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "synth_rng.h"

#define SYNTH_API __attribute__((visibility("default")))

/* Fill out[0..n) with storage units offset..offset+n of tensor (seed,
 * tensor_id), encoded as dtype (a unit is one element; one byte of two
 * elements for SYNTH_MXFP4).  kind/scale/range as in synth_unit().  Returns
 * 0, or -1 on a bad argument. */
SYNTH_API int synth_fill_host(void *out, int dtype, int64_t n, uint64_t seed,
                              uint32_t tensor_id, int64_t offset, int kind, float scale,
                              int32_t range) {
  if (!out || n < 0 || offset < 0) return -1;
  if (dtype < SYNTH_F32 || dtype > SYNTH_E8M0) return -1;
  if (kind != SYNTH_NORMAL && kind != SYNTH_DYADIC) return -1;
  if (kind == SYNTH_DYADIC && range < 0) return -1;
  if (dtype == SYNTH_E8M0 && (range < 1 || range > 253)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t v = synth_unit(dtype, seed, tensor_id, (uint64_t)(offset + i), kind, scale, range);
    if (dtype == SYNTH_F32) ((uint32_t *)out)[i] = v;
    else if (dtype == SYNTH_BF16) ((uint16_t *)out)[i] = (uint16_t)v;
    else ((uint8_t *)out)[i] = (uint8_t)v;
  }
  return 0;
}

/* Raw Philox-4x32-10 block, for known-answer tests of the generator. */
SYNTH_API void synth_philox_host(uint32_t ctr[4], const uint32_t key[2]) {
  synth_philox4x32_10(ctr, key);
}

SYNTH_API int32_t synth_normal_int_host(uint64_t seed, uint32_t tensor_id, uint64_t index) {
  return synth_normal_int(seed, tensor_id, index);
}

SYNTH_API uint16_t synth_bf16_host(float f) { return synth_f32_to_bf16(f); }
SYNTH_API uint8_t synth_e4m3_host(float f) { return synth_f32_to_e4m3(f); }
SYNTH_API uint8_t synth_e2m1_host(float f) { return synth_f32_to_e2m1(f); }

/* Per-block fp32 scales for an fp8 matrix: out[b] = base * (0.75 + 0.5 u_b),
 * u_b uniform in [0,1).  A block scale multiplies every code of its block. */
SYNTH_API int synth_block_scales_host(float *out, int64_t nblocks, uint64_t seed,
                                      uint32_t tensor_id, double base) {
  if (!out || nblocks < 0) return -1;
  for (int64_t b = 0; b < nblocks; ++b) {
    double u = (double)synth_uniform01(seed, tensor_id, (uint64_t)b);
    out[b] = (float)(base * (0.75 + 0.5 * u));
  }
  return 0;
}

/* Zipf(s) per-expert logit offsets b_e = ln(E * p_e), p_e = (e+1)^-s / H,
 * H = sum_{r=1..E} r^-s.  Under these offsets expert e is favoured in
 * proportion to p_e when logits are otherwise exchangeable. */
SYNTH_API int synth_zipf_offsets_host(float *out, int64_t n_experts, double s) {
  if (!out || n_experts <= 0) return -1;
  double h = 0.0;
  for (int64_t r = 1; r <= n_experts; ++r) h += pow((double)r, -s);
  for (int64_t e = 0; e < n_experts; ++e) {
    double p = pow((double)(e + 1), -s) / h;
    out[e] = (float)log((double)n_experts * p);
  }
  return 0;
}

/* Routing indices for dispatch tests: for each of bt tokens, k distinct
 * expert ids in [0, n_experts), ascending.  With hot > 0 the draws are
 * restricted, with probability 1/2 each, to the first `hot` experts, which
 * skews the per-expert counts and leaves some experts empty.  Returns -1 on a
 * bad argument. */
SYNTH_API int synth_routing_host(int32_t *idx, int64_t bt, int64_t k, int64_t n_experts,
                                 uint64_t seed, uint32_t tensor_id, int64_t hot) {
  if (!idx || bt < 0 || k <= 0 || k > n_experts || hot < 0 || hot > n_experts) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < bt; ++t) {
    int32_t *row = idx + t * k;
    int64_t have = 0;
    uint64_t ctr = (uint64_t)t << 20;
    while (have < k) {
      uint32_t r[4];
      synth_draw(seed, tensor_id, ctr++, r);
      int64_t pool = n_experts;
      if (hot > 0 && (r[1] & 1u) && hot >= k) pool = hot;
      int32_t e = (int32_t)(r[0] % (uint32_t)pool);
      int dup = 0;
      for (int64_t j = 0; j < have; ++j) dup |= (row[j] == e);
      if (dup) continue;
      /* insertion keeps the row ascending */
      int64_t j = have;
      while (j > 0 && row[j - 1] > e) { row[j] = row[j - 1]; --j; }
      row[j] = e;
      ++have;
    }
  }
  return 0;
}
