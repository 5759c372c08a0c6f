/*
 * attn_mfma_rate.h -- measurement helper shipped with the attention library:
 * the sustained rate of the matrix cores on this GPU for the instruction the
 * eight-wave attention kernel spends its time in (v_mfma_f32_16x16x32_bf16),
 * on operands the caller chooses.
 *
 * Why: the published dense bf16 peak assumes the top clock, but under a
 * sustained MFMA load the clock is set by power, and power depends on how
 * much the operand bits toggle. A kernel's fraction of the published peak
 * therefore mixes its own efficiency with the chip's power limit; timing
 * this pure MFMA stream on the same data distribution separates the two.
 *
 * attn_mfma_rate enqueues one kernel of `workgroups` workgroups of 256
 * threads (4 waves). Every thread reads 128 bytes of bf16 operands from
 * `operands` (thread t at byte offset 128 * t: four A and four B
 * fragments) and then issues `iters` rounds of 32 MFMAs (eight independent
 * accumulators in VGPRs, as in the attention kernel) from registers, with
 * no memory access in the loop; it finally writes one float per thread to
 * `sink` so that nothing is optimised away. FLOPs per launch =
 * workgroups * 4 * iters * 32 * 16384.
 *
 *   operands : device, 16-byte aligned, workgroups * 256 * 128 bytes, read only
 *   sink     : device float32, workgroups * 256 elements, written
 *   stream   : hipStream_t; NULL means the default stream
 * Ownership and errors as for attn_fwd (include/attn_fwd.h): caller-owned
 * device buffers, no allocation, no synchronisation; returns ATTN_OK,
 * ATTN_ERR_NULL, ATTN_ERR_ALIGN, ATTN_ERR_SHAPE (workgroups or iters < 1,
 * or workgroups * 256 threads above 2^31 - 1) or ATTN_ERR_LAUNCH.
 */
#ifndef ATTN_MFMA_RATE_H
#define ATTN_MFMA_RATE_H

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

ATTN_API int attn_mfma_rate(const void* operands, float* sink, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MFMA_RATE_H */
