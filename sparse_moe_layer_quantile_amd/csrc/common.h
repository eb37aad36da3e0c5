// common.h -- shared device helpers of the gfx950 MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_API extern "C" __attribute__((visibility("default")))

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

namespace moe {

// Launch returning that launch's own status (hipGetLastError would also
// report errors left behind by earlier runtime calls of the process).
template <typename T>
struct launch_arg {
  using type = T;
};
template <typename... KArgs>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                                hipStream_t stream, typename launch_arg<KArgs>::type... args) {
  void *argv[] = {static_cast<void *>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, stream);
}

// ---- bf16 storage ------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// Round to nearest even; finite inputs only.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---- fp8 e4m3fn (OCP) -> fp32, from the format definition --------------------
// 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds the
// subnormals m * 2^-9.  NaN (S.1111.111) is not expected in weights.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t em = code & 0x7Fu;
  float v;
  if (em >= 0x08u) {
    v = __uint_as_float(((em >> 3) + 120u) << 23 | (em & 7u) << 20);
  } else {
    v = (float)em * (1.0f / 512.0f);
  }
  return __uint_as_float(__float_as_uint(v) | sign);
}

// ---- OCP MX FP8 (e4m3 elements, E8M0 scale per 32) ---------------------------
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

// Shared exponent of an MX block from its largest magnitude (OCP MX v1.0):
// floor(log2 amax) - 8 (8 = the largest e4m3 exponent), clamped to [-127, 127];
// -127 for an all-zero block.  The E8M0 scale byte is shared + 127.
__device__ __forceinline__ int mx8_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int e = (int)(__float_as_uint(amax) >> 23) - 127;  // floor(log2); subnormal: -127
  return max(-127, min(127, e - 8));
}

// ---- elementary functions (from their definitions via exp) ------------------
// exp(x) = 2^(x log2 e) on the hardware exp2 unit.
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }
// sigmoid(x) = 1 / (1 + e^-x)
__device__ __forceinline__ float sigmoid_f(float x) { return rcp_fast(1.0f + exp_fast(-x)); }
// tanh(x) = sign(x) (1 - e^-2|x|) / (1 + e^-2|x|)
__device__ __forceinline__ float tanh_f(float x) {
  const float e = exp_fast(-2.0f * fabsf(x));
  return copysignf((1.0f - e) * rcp_fast(1.0f + e), x);
}
// SiTU-GLU factors: phi(g) = sigmoid(g) beta tanh(g / beta), psi(u) = beta_u tanh(u / beta_u)
__device__ __forceinline__ float situ_phi(float g, float beta, float inv_beta) {
  return sigmoid_f(g) * beta * tanh_f(g * inv_beta);
}
__device__ __forceinline__ float situ_psi(float u, float beta_u, float inv_beta_u) {
  return beta_u * tanh_f(u * inv_beta_u);
}
__device__ __forceinline__ float situ(float g, float u, float beta, float inv_beta,
                                      float beta_u, float inv_beta_u) {
  return situ_phi(g, beta, inv_beta) * situ_psi(u, beta_u, inv_beta_u);
}

// Order-preserving map of an fp32 value to uint32 (larger value -> larger
// key); -0 is folded onto +0 so that equal values give equal keys.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace moe
