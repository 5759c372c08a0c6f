// C ABI entry points: argument validation (pure host code) and the launch.
#include "attn_fwd.h"

#include <cmath>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "attn_fwd_launch.h"

namespace {

constexpr int kHeadDim = 128;
constexpr int kBlockM = 128;
// Launch limit: the total thread count of a 1-D grid must stay below 2^32.
constexpr int64_t kMaxThreads = (int64_t(1) << 32) - 1;

bool basic_shape_ok(int B, int H, int S, int D) {
  return D == kHeadDim && B >= 1 && H >= 1 && S >= kBlockM && S % kBlockM == 0;
}

bool grid_ok(int B, int H, int S, int variant) {
  return attn_detail::launch_threads(B, H, S, variant) <= kMaxThreads;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, uint64_t a_bytes, const void* b, uint64_t b_bytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

// Validation for a given resolved variant (AUTO resolves to the pick).
int check_with_variant(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       int B, int H, int S, int D, float scale, int variant) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (!basic_shape_ok(B, H, S, D)) return ATTN_ERR_SHAPE;
  if (variant == ATTN_VARIANT_AUTO) variant = attn_detail::pick_variant(B, H, S);
  if (!grid_ok(B, H, S, variant)) return ATTN_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_SCALE;
  const uint64_t rows = uint64_t(B) * uint64_t(H) * uint64_t(S);
  const uint64_t tensor_bytes = rows * kHeadDim * 2;
  const uint64_t lse_bytes = rows * 4;
  if (overlaps(o, tensor_bytes, q, tensor_bytes) || overlaps(o, tensor_bytes, k, tensor_bytes) ||
      overlaps(o, tensor_bytes, v, tensor_bytes) || overlaps(lse, lse_bytes, q, tensor_bytes) ||
      overlaps(lse, lse_bytes, k, tensor_bytes) || overlaps(lse, lse_bytes, v, tensor_bytes) ||
      overlaps(lse, lse_bytes, o, tensor_bytes))
    return ATTN_ERR_OVERLAP;
  return ATTN_OK;
}

}  // namespace

extern "C" ATTN_API int attn_fwd_check(const void* q, const void* k, const void* v, const void* o,
                                       const float* lse, int B, int H, int S, int D, float scale) {
  return check_with_variant(q, k, v, o, lse, B, H, S, D, scale, ATTN_VARIANT_AUTO);
}

extern "C" ATTN_API int attn_fwd_pick(int B, int H, int S) { return attn_detail::pick_variant(B, H, S); }

extern "C" ATTN_API int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int S, int D, float scale, int variant, void* stream) {
  if (variant != ATTN_VARIANT_AUTO && variant != ATTN_VARIANT_TILE128 &&
      variant != ATTN_VARIANT_PAIR256 && variant != ATTN_VARIANT_PAIR256_EXP2EMU &&
      variant != ATTN_VARIANT_PAIR128)
    return ATTN_ERR_VARIANT;
  const int status = check_with_variant(q, k, v, o, lse, B, H, S, D, scale, variant);
  if (status != ATTN_OK) return status;
  attn_detail::Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.S = S;
  p.scale = scale;
  p.variant = variant == ATTN_VARIANT_AUTO ? attn_detail::pick_variant(B, H, S) : variant;
  const hipError_t err = attn_detail::launch(p, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int S, int D, float scale, void* stream) {
  return attn_fwd_variant(q, k, v, o, lse, B, H, S, D, scale, ATTN_VARIANT_AUTO, stream);
}

extern "C" ATTN_API const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE:
      return "unsupported shape (need D == 128, S >= 128, S % 128 == 0, B, H >= 1, under 2^32 threads)";
    case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_OVERLAP: return "output buffer overlaps another buffer";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_VARIANT: return "unknown kernel variant";
    default: return "unknown status";
  }
}
