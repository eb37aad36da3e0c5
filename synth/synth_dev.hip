// synth_dev.hip -- device (gfx950) generator of seeded synthetic layer inputs.
//
// Writes a tensor straight into device memory with the same bits as
// synth_fill_host() in synth_host.c (both expand synth_rng.h), so a
// 60 GB layer is generated in HBM without a host copy, while the CPU side can
// regenerate any slice of it.  Holds no arithmetic of the MoE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_rng.h"

#define SYNTH_API extern "C" __attribute__((visibility("default")))

template <int DT>
__global__ void __launch_bounds__(256) synth_fill_kernel(void *out, int64_t n, uint64_t seed,
                                                         uint32_t tensor_id, int64_t offset,
                                                         int kind, float scale, int32_t range) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t v = synth_unit(DT, seed, tensor_id, (uint64_t)(offset + i), kind, scale, range);
    if (DT == SYNTH_F32) ((uint32_t *)out)[i] = v;
    else if (DT == SYNTH_BF16) ((uint16_t *)out)[i] = (uint16_t)v;
    else ((uint8_t *)out)[i] = (uint8_t)v;
  }
}

// Device twin of synth_fill_host.  `out` is a device pointer with room for n
// storage units of dtype.  Enqueued on `stream`; returns 0, -1 on a bad argument,
// -1000 - (hipError_t) if the launch failed.
SYNTH_API int synth_fill_device(void *out, int dtype, int64_t n, uint64_t seed,
                                uint32_t tensor_id, int64_t offset, int kind, float scale,
                                int32_t range, hipStream_t stream) {
  if (n < 0 || offset < 0) return -1;
  if (n == 0) return 0;
  if (!out) return -1;
  if (kind != SYNTH_NORMAL && kind != SYNTH_DYADIC) return -1;
  if (kind == SYNTH_DYADIC && range < 0) return -1;
  if (dtype == SYNTH_E8M0 && (range < 1 || range > 253)) return -1;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  void (*kern)(void *, int64_t, uint64_t, uint32_t, int64_t, int, float, int32_t);
  switch (dtype) {
    case SYNTH_F32: kern = synth_fill_kernel<SYNTH_F32>; break;
    case SYNTH_BF16: kern = synth_fill_kernel<SYNTH_BF16>; break;
    case SYNTH_FP8E4M3: kern = synth_fill_kernel<SYNTH_FP8E4M3>; break;
    case SYNTH_MXFP4: kern = synth_fill_kernel<SYNTH_MXFP4>; break;
    case SYNTH_E8M0: kern = synth_fill_kernel<SYNTH_E8M0>; break;
    default: return -1;
  }
  // hipLaunchKernel reports this launch's own status (hipGetLastError would
  // also report errors left behind by earlier runtime calls of the process)
  void *args[] = {&out, &n, &seed, &tensor_id, &offset, &kind, &scale, &range};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3((unsigned)blocks),
                                       dim3(256), args, 0, stream);
  return e == hipSuccess ? 0 : -1000 - (int)e;
}
