// Sustained-rate stream of v_mfma_f32_32x32x16_bf16 (declared in
// include/attn_mfma_rate.h): four independent accumulators, operands held in
// registers, no memory access in the loop.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_mfma_rate.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void mfma_rate_kernel(const bf16x8* __restrict__ src,
                                                        float* __restrict__ sink, int iters) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[t * 8 + i];
    b[i] = src[t * 8 + 4 + i];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + 1) & 3], b[i], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + 2) & 3], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + 3) & 3], b[(i + 1) & 3], c3, 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[t] = s;
}

}  // namespace

extern "C" int attn_mfma_rate(const void* operands, float* sink, int workgroups, int iters,
                              void* stream) {
  if (!operands || !sink) return ATTN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(operands) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return ATTN_ERR_ALIGN;
  if (workgroups < 1 || iters < 1 || int64_t(workgroups) * 256 > INT32_MAX) return ATTN_ERR_SHAPE;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const bf16x8*>(operands), sink, iters);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
