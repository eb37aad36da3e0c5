// quant.hip -- MX FP8 quantisation of activations: the inputs of the routed
// experts' GEMMs on the block-scaled MFMA path (x_lat for gate/up, h for down).
//
// OCP Microscaling Formats (MX) Specification v1.0, the conversion of a vector
// of scalars to an MX block: per 32 consecutive elements the shared exponent is
// floor(log2(max |x|)) - 8 (8 = the largest E4M3 exponent), clamped to
// [-127, 127] (-127 for an all-zero block), stored as the E8M0 code shared + 127;
// each element becomes x / 2^shared rounded to the nearest E4M3 value, ties to
// even, saturating at 448.  The scaling by a power of two is exact, so the
// codes depend only on the bf16 input.
//
// One thread per 8 consecutive elements (a 16-byte load), four threads per
// block; the block maximum is exchanged within the four lanes.
#include "common.h"
#include "kernels.h"

namespace moe {

// Nearest E4M3 code of a finite fp32 value (OCP e4m3fn: bias 7, 3 mantissa
// bits, largest 448), ties to even, saturating.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |v| >= 448
  const int e = (int)(a >> 23) - 127;
  if (e < -126) return sign;  // zero or fp32 subnormal: far below half the least E4M3 step
  const uint32_t f = a & 0x7FFFFFu;
  if (e < -6) {
    // subnormal E4M3: |v| / 2^-9 rounded to an integer in [0, 8] (8 = least normal)
    const uint32_t m = f | 0x800000u;  // |v| = m 2^(e - 23)
    const int shift = 14 - e;          // |v| / 2^-9 = m / 2^shift
    if (shift > 24) return sign;
    const uint32_t q = (m + (1u << (shift - 1)) - 1u + ((m >> shift) & 1u)) >> shift;
    return sign | q;
  }
  uint32_t mant = (f + 0x7FFFFu + ((f >> 20) & 1u)) >> 20;  // 23 -> 3 bits, ties to even
  int eb = e + 7;
  if (mant == 8u) {
    mant = 0u;
    ++eb;
  }
  const uint32_t code = ((uint32_t)eb << 3) | mant;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__global__ void __launch_bounds__(256) mx8_quant_kernel(const uint16_t *__restrict__ x,
                                                        int64_t n8, uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8-element group
  const bool live = t < n8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (live) v = reinterpret_cast<const uint4 *>(x)[t];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_to_f32((uint16_t)(w[q] & 0xFFFFu));
    f[2 * q + 1] = bf16_to_f32((uint16_t)(w[q] >> 16));
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * q]), fabsf(f[2 * q + 1])));
  }
  // the four lanes of a 32-element block (groups of 4 consecutive lanes)
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  int shared = -127;
  if (amax > 0.0f) {
    const int e = (int)(__float_as_uint(amax) >> 23) - 127;  // floor(log2 amax); subnormal: -127
    shared = max(-127, min(127, e - 8));
  }
  if (!live) return;
  const float inv = __uint_as_float((uint32_t)(127 - shared) << 23);  // 2^-shared
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3_sat(f[i] * inv) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3_sat(f[4 + i] * inv) << (8 * i);
  reinterpret_cast<uint2 *>(codes)[t] = make_uint2(lo, hi);
  if ((t & 3) == 0) scales[t >> 2] = (uint8_t)(shared + 127);
}

hipError_t launch_mx8_quant(const void *x, int64_t n, uint8_t *codes, uint8_t *scales,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 32) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  return launch_kernel(mx8_quant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(x), n8, codes, scales);
}

}  // namespace moe
