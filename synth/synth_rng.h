/*
 * synth_rng.h -- seeded, counter-based generation of synthetic layer inputs.
 *
 * This header is the one piece of code that the host generator
 * (synth_host.c, built by gcc) and the device generator (synth_dev.hip,
 * built by hipcc) have in common.  It holds no arithmetic of the MoE layer:
 * only a random-number generator and the encodings of its draws into the
 * storage formats the layer reads (fp32, bf16, fp8 e4m3fn, OCP MX FP4 E2M1
 * with E8M0 block scales).  Everything is
 * integer arithmetic or a single IEEE fp32 multiply, so the host and the
 * device produce bit-identical tensors.
 *
 * Generator: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), key = 64-bit seed, counter =
 * (flat element index lo, hi, tensor id, 0).
 *
 * "Normal" draw: Irwin-Hall sum of the eight 16-bit halves of one Philox
 * output, centred: v = 2*sum - 8*65535, an even integer in
 * [-524280, 524280] with standard deviation NORMAL_INT_STD.  The stored value
 * is (float)v * scale (one correctly rounded fp32 multiply), so a tensor
 * drawn with scale = sigma / NORMAL_INT_STD has standard deviation sigma
 * and |value| <= 4.899 sigma.
 *
 * "Dyadic" draw: an integer k uniform in [-range, range] times a
 * power-of-two scale.  Dot products of such tensors are exact in fp32,
 * which makes router logits identical on every accumulation order.
 */
#ifndef SYNTH_RNG_H
#define SYNTH_RNG_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

/* SYNTH_MXFP4 fills bytes of two E2M1 codes each: byte i holds tensor
 * elements 2i (low nibble) and 2i + 1 (high nibble).  SYNTH_E8M0 fills block
 * scale codes centre + u, u uniform in {-1, 0, 1}. */
enum { SYNTH_F32 = 0, SYNTH_BF16 = 1, SYNTH_FP8E4M3 = 2, SYNTH_MXFP4 = 3, SYNTH_E8M0 = 4 };
enum { SYNTH_NORMAL = 0, SYNTH_DYADIC = 1 };

/* sqrt(8 * 4 * (65536^2 - 1) / 12): std of v = 2*sum(8 uniform u16) - 8*65535 */
#define SYNTH_NORMAL_INT_STD 107022.329313
#define SYNTH_NORMAL_INT_MAX 524280

SYNTH_FN uint32_t synth_mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) >> 32);
}

/* Philox-4x32 with 10 rounds.  ctr[4] in/out, key[2] in. */
SYNTH_FN void synth_philox4x32_10(uint32_t ctr[4], const uint32_t key_in[2]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t k0 = key_in[0], k1 = key_in[1];
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    uint32_t hi0 = synth_mulhi32(M0, c0), lo0 = M0 * c0;
    uint32_t hi1 = synth_mulhi32(M1, c2), lo1 = M1 * c2;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  ctr[0] = c0; ctr[1] = c1; ctr[2] = c2; ctr[3] = c3;
}

SYNTH_FN void synth_draw(uint64_t seed, uint32_t tensor_id, uint64_t index,
                         uint32_t out[4]) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  out[0] = (uint32_t)index;
  out[1] = (uint32_t)(index >> 32);
  out[2] = tensor_id;
  out[3] = 0u;
  synth_philox4x32_10(out, key);
}

/* Centred Irwin-Hall integer of the draw (see header comment). */
SYNTH_FN int32_t synth_normal_int(uint64_t seed, uint32_t tensor_id, uint64_t index) {
  uint32_t r[4];
  synth_draw(seed, tensor_id, index, r);
  int32_t s = 0;
  for (int i = 0; i < 4; ++i) s += (int32_t)(r[i] & 0xFFFFu) + (int32_t)(r[i] >> 16);
  return 2 * s - 8 * 65535;
}

/* Integer uniform in [-range, range]. */
SYNTH_FN int32_t synth_dyadic_int(uint64_t seed, uint32_t tensor_id, uint64_t index,
                                  int32_t range) {
  uint32_t r[4];
  synth_draw(seed, tensor_id, index, r);
  uint32_t span = (uint32_t)(2 * range + 1);
  return (int32_t)(r[0] % span) - range;
}

/* Uniform in [0, 1) with 24 random bits (exact in fp32). */
SYNTH_FN float synth_uniform01(uint64_t seed, uint32_t tensor_id, uint64_t index) {
  uint32_t r[4];
  synth_draw(seed, tensor_id, index, r);
  return (float)(r[0] >> 8) * (1.0f / 16777216.0f);
}

SYNTH_FN uint32_t synth_f32_bits(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  return c.u;
}

/* fp32 -> bf16, round to nearest even (finite inputs). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  uint32_t u = synth_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp32 -> OCP fp8 e4m3fn (bias 7, no infinities, 0x7F is NaN, max 448),
 * round to nearest even, saturating to +-448 (finite inputs). */
SYNTH_FN uint8_t synth_f32_to_e4m3(float f) {
  uint32_t u = synth_f32_bits(f);
  uint32_t sign = (u >> 24) & 0x80u;
  u &= 0x7FFFFFFFu;
  if (u == 0u) return (uint8_t)sign;
  int32_t ex = (int32_t)(u >> 23) - 127;
  uint32_t code;
  if (ex < -6) {
    /* subnormal range: value = q * 2^-9, q in [0, 8] */
    uint32_t m = (u & 0x7FFFFFu) | 0x800000u; /* value = m * 2^(ex-23) */
    int32_t shift = 14 - ex;                   /* q = m * 2^(ex-14) */
    if (shift > 25) {
      code = 0u;
    } else {
      uint32_t half = 1u << (shift - 1);
      uint32_t q = (m + half - 1u + ((m >> shift) & 1u)) >> shift;
      code = q; /* q == 8 encodes the smallest normal, 2^-6 */
    }
  } else {
    uint32_t m23 = u & 0x7FFFFFu;
    uint32_t mant = (m23 + 0x7FFFFu + ((m23 >> 20) & 1u)) >> 20;
    int32_t eb = ex + 7;
    if (mant == 8u) { mant = 0u; eb += 1; }
    if (eb > 15 || (eb == 15 && mant == 7u)) code = 0x7Eu; /* saturate to 448 */
    else code = ((uint32_t)eb << 3) | mant;
  }
  return (uint8_t)(sign | code);
}

/* fp32 -> OCP MX FP4 E2M1 code (sign bit 3, exponent bits 2:1 with bias 1,
 * mantissa bit 0; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or
 * NaN), round to nearest even, saturating to +-6 (finite inputs). */
SYNTH_FN uint8_t synth_f32_to_e2m1(float f) {
  uint32_t u = synth_f32_bits(f);
  uint32_t sign = (u >> 28) & 0x8u;
  u &= 0x7FFFFFFFu;
  if (u == 0u) return (uint8_t)sign;
  int32_t ex = (int32_t)(u >> 23) - 127;
  uint32_t code;
  if (ex > 2) {
    code = 0x7u; /* 8 and above */
  } else if (ex < 0) {
    /* below 1: value = q * 2^-1, q in [0, 2]; q == 2 is code 2 (1.0) */
    uint32_t m = (u & 0x7FFFFFu) | 0x800000u; /* value = m * 2^(ex-23) */
    int32_t shift = 22 - ex;                   /* q = m * 2^(ex-22) */
    if (shift > 25) {
      code = 0u;
    } else {
      uint32_t half = 1u << (shift - 1);
      code = (m + half - 1u + ((m >> shift) & 1u)) >> shift;
    }
  } else {
    uint32_t m23 = u & 0x7FFFFFu;
    uint32_t mant = (m23 + 0x1FFFFFu + ((m23 >> 22) & 1u)) >> 22;
    int32_t eb = ex + 1;
    if (mant == 2u) { mant = 0u; eb += 1; }
    code = eb > 3 ? 0x7u : (((uint32_t)eb << 1) | mant);
  }
  return (uint8_t)(sign | code);
}

/* E8M0 block-scale code of draw `index`: centre + u, u uniform in {-1, 0, 1}. */
SYNTH_FN uint8_t synth_e8m0(uint64_t seed, uint32_t tensor_id, uint64_t index, int32_t centre) {
  return (uint8_t)(centre + synth_dyadic_int(seed, tensor_id, index, 1));
}

/* The value of element `index` of a tensor as an fp32 number. */
SYNTH_FN float synth_value(uint64_t seed, uint32_t tensor_id, uint64_t index, int kind,
                           float scale, int32_t range) {
  if (kind == SYNTH_DYADIC)
    return (float)synth_dyadic_int(seed, tensor_id, index, range) * scale;
  return (float)synth_normal_int(seed, tensor_id, index) * scale;
}

/* Storage unit i (of a fill starting at unit `offset`) of a tensor of the
 * given dtype, as raw bits in the low bytes of the result.  kind/scale/range
 * as in synth_value(); for SYNTH_E8M0, range is the centre code. */
SYNTH_FN uint32_t synth_unit(int dtype, uint64_t seed, uint32_t tensor_id, uint64_t unit,
                             int kind, float scale, int32_t range) {
  if (dtype == SYNTH_E8M0) return synth_e8m0(seed, tensor_id, unit, range);
  if (dtype == SYNTH_MXFP4) {
    uint32_t lo = synth_f32_to_e2m1(synth_value(seed, tensor_id, 2 * unit, kind, scale, range));
    uint32_t hi = synth_f32_to_e2m1(synth_value(seed, tensor_id, 2 * unit + 1, kind, scale, range));
    return lo | (hi << 4);
  }
  float v = synth_value(seed, tensor_id, unit, kind, scale, range);
  if (dtype == SYNTH_F32) return synth_f32_bits(v);
  if (dtype == SYNTH_BF16) return synth_f32_to_bf16(v);
  return synth_f32_to_e4m3(v);
}

#endif /* SYNTH_RNG_H */
