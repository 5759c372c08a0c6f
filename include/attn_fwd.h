/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) dense attention forward.
 *
 * Operation (the "B200 attention kernel from scratch to ~SOTA in 60
 * figures" article, Chapter 1 "ii. Work parallelization" and section B):
 * for every batch b, head h and query row i,
 *
 *     O[b,h,i,:] = sum_j softmax_j(scale * q_i . k_j) * v_j
 *
 * dense (no mask), non-causal, bf16 inputs, head_dim 128. The kernel walks
 * the keys tile by tile with an online softmax (article, Chapter 1 section
 * B; Chapter 8 for the base-2 exponent with the scale folded in; Chapter
 * 11 for the lazily skipped rescale), so the S x S score matrix never
 * exists in memory. It also writes the natural-log log-sum-exp of each
 * row's softmax denominator, lse[b,h,i] = ln sum_j exp(scale * q_i . k_j),
 * which the article does not define (it is the quantity a split over keys
 * needs to merge partial results).
 *
 * Layout: q, k, v and o are contiguous row-major [B, H, S, D] arrays of
 * bf16 (2 bytes each, D innermost); lse is a contiguous [B, H, S] array of
 * float32. Index arithmetic is 64-bit.
 *
 * Ownership: every pointer is a device pointer owned by the caller. The
 * library allocates nothing, keeps no state between calls and never
 * synchronises: attn_fwd enqueues one kernel on `stream` and returns, so a
 * caller may also capture it into a HIP graph. q, k, v are only read;
 * every element of o and lse is written.
 *
 * Errors: each function returns an attn_status code; nothing is printed
 * and nothing throws. A fault inside the kernel is reported by the HIP
 * runtime at the caller's next synchronisation on that stream.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

/* The library is built with hidden symbol visibility; exactly the functions
 * declared with ATTN_API in this directory's headers are exported. */
#if defined(__GNUC__) || defined(__clang__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,       /* a pointer argument is NULL */
  ATTN_ERR_SHAPE = 2,      /* D != 128, S < 128, S % 128 != 0, B < 1, H < 1, or the
                              launch of the kernel variant used would have 2^32 or
                              more threads (about B*H*S >= 2^32 for every variant) */
  ATTN_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned */
  ATTN_ERR_SCALE = 4,      /* scale is not finite or not > 0 (the row max is taken
                              over raw scores and scaled afterwards, which needs a
                              positive scale) */
  ATTN_ERR_OVERLAP = 5,    /* o or lse overlaps q, k, v or each other */
  ATTN_ERR_LAUNCH = 6,     /* the HIP runtime rejected the kernel launch */
  ATTN_ERR_VARIANT = 7     /* unknown kernel variant */
};

/*
 * Kernel variants. All compute the same operation to the same tolerance;
 * they differ in how work is laid out on the GPU.
 *   ATTN_VARIANT_AUTO    : what attn_fwd uses (see attn_fwd_pick)
 *   ATTN_VARIANT_TILE128 : 4-wave workgroups, one 128-row query tile each
 *   ATTN_VARIANT_PAIR256 : 8-wave workgroups holding two 128-row query
 *                          tiles of one head that share every K/V tile, the
 *                          two 4-wave groups phase-shifted so one runs its
 *                          matrix products while the other runs its softmax
 *   ATTN_VARIANT_PAIR256_EXP2EMU : PAIR256 with one exponential in four
 *                          computed by a polynomial on the FMA pipe instead
 *                          of the exponent unit (the article's Chapter 9
 *                          "software approximations"); for measurement,
 *                          never picked by attn_fwd
 *   ATTN_VARIANT_PAIR128 : PAIR256's 8-wave workgroups with two 64-row
 *                          query tiles, for mid-sized grids
 */
enum attn_variant {
  ATTN_VARIANT_AUTO = 0,
  ATTN_VARIANT_TILE128 = 1,
  ATTN_VARIANT_PAIR256 = 2,
  ATTN_VARIANT_PAIR256_EXP2EMU = 3,
  ATTN_VARIANT_PAIR128 = 4
};

/*
 * Dense attention forward.
 *   q, k, v : bf16 [B,H,S,D] inputs (device, 16-byte aligned, read only)
 *   o       : bf16 [B,H,S,D] output (device, 16-byte aligned)
 *   lse     : fp32 [B,H,S] output, natural-log log-sum-exp per query row,
 *             ln sum_j exp(scale * q_i . k_j) (see "Accuracy" below)
 *   B, H, S : batch, heads, sequence length (queries = keys = S)
 *   D       : head dimension, must be 128
 *   scale   : softmax scale applied to q.k, finite and > 0 (usually 1/sqrt(D));
 *             the kernels work in fp32 on scale * log2(e) * q.k, so every such
 *             product must stay below 2^30 in magnitude (about 1e9): beyond
 *             that, the fp32 rounding of a scaled score (its ulp exceeds 128
 *             base-2 units) can push an exponent past the fp32 range and the
 *             output becomes non-finite. Well below that limit, the fp32
 *             rounding of the scores themselves already bounds the accuracy
 *             of rows whose largest scores nearly tie.
 *   stream  : hipStream_t to enqueue on; NULL means the default stream
 * Inputs must be finite; NaN or Inf in q, k or v gives unspecified output.
 * Returns ATTN_OK or an error code; on error nothing is enqueued (except
 * ATTN_ERR_LAUNCH, where the runtime refused the launch).
 *
 * Accuracy. The unnormalised probabilities p_j are rounded to bf16 before
 * they multiply v (as in the article, Chapter 1 section B), and the row sum
 * adds these same rounded values (the article adds the unrounded ones), so
 * o is a convex combination of the rows of v with weights off by at most
 * 2^-8 relative each. lse is taken from
 * that same sum: its absolute error is at most -ln(1 - 2^-8) ~= 3.9e-3 (the
 * worst case, reached when one or a few keys carry nearly all of a row's
 * weight and their p round the same way), plus fp32 rounding of order
 * 1e-6 * |lse|. Where many keys share the weight their rounding errors
 * cancel: on normally distributed inputs the error is of order 1e-5 to 1e-4
 * relative. A caller that merges partial results by their lse (a split
 * over keys) sees the merge weights off by at most about 0.4%, the same
 * order as the bf16 rounding of o itself.
 * Range. The PAIR variants keep each row's running base 47 base-2 units
 * above the row max at its last move, so their unnormalised p lie in
 * [2^-47, 2) for the largest key of a row while the fp32 ulp of the scaled
 * scores is below that margin (|scale * q.k| below about 2^28), and below
 * 2^17 up to the 2^30 limit: the fp32 accumulator of o stays below
 * 2 * S * max|v| (2^17 * S * max|v| near the limit), and for |v| below about
 * 2^-79 the products p * v leave the normal range, where o keeps only its
 * absolute accuracy. TILE128 keeps p in [1, 2^16) for the largest key (up
 * to 2^64 near the limit), so its accumulator stays below 2^16 * S * max|v|.
 */
ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, float scale, void* stream);

/*
 * attn_fwd with an explicit kernel variant (enum attn_variant); the same
 * arguments, layout, ownership and errors as attn_fwd, plus
 * ATTN_ERR_VARIANT for an unknown variant. For tests and tuning.
 */
ATTN_API int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S, int D, float scale, int variant, void* stream);

/*
 * The variant attn_fwd picks for a shape (pure host code): PAIR256 when its
 * grid of 128-row tile pairs has at least 256 workgroups (unless that grid
 * would reach 2^32 threads, then TILE128), else PAIR128 when its grid of
 * 64-row tile pairs has at least 16, else TILE128.
 * Returns ATTN_VARIANT_TILE128, ATTN_VARIANT_PAIR128 or ATTN_VARIANT_PAIR256.
 */
ATTN_API int attn_fwd_pick(int B, int H, int S);

/*
 * The argument validation of attn_fwd on its own: pure host code that
 * touches no device memory and needs no GPU. Returns the status attn_fwd
 * would return before launching.
 */
ATTN_API int attn_fwd_check(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, int B, int H, int S, int D, float scale);

/* A static, human-readable name for a status code (never NULL). */
ATTN_API const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
