// Internal interface between the C ABI (validation) and the HIP kernel launch.
#pragma once

#include <hip/hip_runtime_api.h>

namespace attn_detail {

constexpr int kThreads = 256;  // one workgroup = 4 wave64s, 32 query rows each

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, S;
  float scale;
};

// Enqueues the forward kernel on `stream`; arguments are already validated.
hipError_t launch(const Params& p, hipStream_t stream);

}  // namespace attn_detail
