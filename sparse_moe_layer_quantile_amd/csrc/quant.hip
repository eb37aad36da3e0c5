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
  const int shared = mx8_shared_exp(amax);
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
