// Internal interface between the C ABI (validation) and the HIP kernel launch.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

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
  int variant;  // TILE128, PAIR256, PAIR256_EXP2EMU or PAIR128 (resolved, never AUTO)
};

// The variant chosen for a shape when the caller leaves it to the library.
int pick_variant(int B, int H, int S);

// Threads of the launch a resolved variant makes for this shape
// (workgroups x workgroup size); the hardware limit is 2^32 - 1.
int64_t launch_threads(int B, int H, int S, int variant);

// Enqueues the forward kernel on `stream`; arguments are already validated.
hipError_t launch(const Params& p, hipStream_t stream);

}  // namespace attn_detail
