// Sustained-rate stream of v_mfma_f32_16x16x32_bf16 (declared in
// include/attn_mfma_rate.h): eight independent accumulators held in VGPRs
// through tied operands (as the attention kernel holds O), operands in
// registers, no memory access in the loop.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_mfma_rate.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
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
  f32x4 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                     : "+v"(c[i])
                     : "v"(a[(i + r) & 3]), "v"(b[(i + 2 * r) & 3]));
  }
  // the results are read next by VALU code: wait out the MFMA write-back
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]),
               "+v"(c[5]), "+v"(c[6]), "+v"(c[7]));
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  sink[t] = s;
}

}  // namespace

extern "C" ATTN_API int attn_mfma_rate(const void* operands, float* sink, int workgroups, int iters,
                              void* stream) {
  if (!operands || !sink) return ATTN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(operands) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return ATTN_ERR_ALIGN;
  if (workgroups < 1 || iters < 1 || int64_t(workgroups) * 256 > INT32_MAX) return ATTN_ERR_SHAPE;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const bf16x8*>(operands), sink, iters);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
