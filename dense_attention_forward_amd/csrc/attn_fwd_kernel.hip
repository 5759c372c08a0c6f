// Dense, non-causal, bf16, head_dim-128 attention forward for gfx950 (MI355X).
//
// Method: "B200 attention kernel from scratch to ~SOTA in 60 figures",
// Chapter 1 (one workgroup per 128-row output tile, a sequential K/V loop
// inside it, online softmax of section B), Chapter 8 (base-2 exponent with
// scale*log2(e) folded into the score scale; the max is taken over raw
// scores and scaled once), Chapter 11 (the O accumulator is rescaled only
// when a row's max grows past a threshold, decided per wave; the article's
// threshold is 8 in base-2 units; the four-wave kernel uses 16, the
// eight-wave kernel 48 against a raised base, see kRebaseLog2 and
// kBitRebaseLog2),
// Chapters 6-7 (K and V move through separate double buffers, and the
// next tile's QK^T is issued while the current tile's softmax runs).
//
// Two kernels: attn_fwd_kernel (four waves, one 128-row query tile per
// workgroup, for small grids) and attn_fwd_pingpong_kernel (eight waves in
// two phase-shifted groups, two query tiles sharing each K/V tile; see its
// own comment).
//
// gfx950 mapping (not the article's B200 mapping):
//  * Each wave owns 32 query rows (rows 32w..32w+31 of its group's tile).
//  * Scores are computed transposed, S^T = K . Q^T, on
//    v_mfma_f32_32x32x16_bf16: the accumulator of a 32x32 block gives lane
//    l the column l%32 (one query) and rows 8j + 4*(l/32) + i (keys), so a
//    query's row max and row sum are in-lane plus one exchange between the
//    two half-waves.
//  * O is accumulated transposed too, O^T += V^T . P^T, with P^T taken
//    straight from the score accumulators (converted to bf16): for the
//    16-key step t the B operand of lane l holds keys 16t + 4*(l/32) + 0..3
//    and 16t + 8 + 4*(l/32) + 0..3, and the A operand (V^T) is gathered for
//    the same keys with ds_read_b64_tr_b16, which transposes a 4-key x
//    16-column block across each 16-lane group.
//  * K and V tiles reach LDS by global_load_lds_dwordx4 (no registers): a
//    load writes 64 lanes x 16 bytes contiguously, so each 4-row block of a
//    tile is 1 KB whose 16-byte slots are permuted by choosing which chunk
//    each lane fetches. The permutations make every MFMA operand read a
//    per-lane base plus a compile-time offset and keep LDS bank-conflict
//    free (see k_fill_offset / v_fill_offset).
//  * Workgroups are renumbered so that each XCD (blocks are dispatched to
//    the 8 XCDs round-robin) processes a contiguous range of (b, h, tile)
//    work items, keeping one head's K/V in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "attn_fwd.h"
#include "attn_fwd_launch.h"

namespace attn_detail {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
// Fourth word of a raw buffer resource on gfx9: data format 32 bit (bits
// 18:15 = 4), no swizzle, no thread-id offset; raw byte-offset loads ignore
// the format but it must not be the invalid 0.
constexpr int kBufferWord3 = 0x00020000;

constexpr int kD = 128;         // head dimension
constexpr int kBM = 128;        // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Rebase threshold of the four-wave kernel in base-2 exponent units: a row
// keeps its base until its max exceeds it by this much, so unnormalised P
// stays below 2^16 and O below 2^16 * S * max|V| (fp32 overflows only for
// |V| beyond ~2^80). A rescale of O costs 65 serial VALU instructions; 16
// instead of the article's 8 makes it rare on peaked rows (normal Q and K
// of standard deviation 2 at S = 8192: from 17% of tiles per wave to 0.1%).
constexpr float kRebaseLog2 = 16.0f;
// Rebase threshold of the eight-wave kernel. Its kept base sits
// kBitRebaseLog2 - 1 above the row's max * c at the row's last rebase, so
// every P it computes is below 2 until some score passes the threshold,
// and "P >= 2" is the top exponent bit of the bf16 P (pp_v_phase tests it
// with one OR over all of a wave's P). O then stays below 2 * S * max|V|.
// The price is at the small end: right after a rebase the largest P is
// 2^-47, so products P * V leave fp32's normal range once |V| is under
// about 2^-79 (O keeps its absolute accuracy, not its relative one, for
// such V). A rebase costs this kernel a second pass of exponentials; at 48
// no row of the 4K-16K workloads rebases after its first tile (at 16, 16.9%
// of a wave's tiles on the 16K outlier workload; at 32, 3.7%).
constexpr float kBitRebaseLog2 = 48.0f;

// Tile parameters (compile-time): keys per K/V tile and the waves per SIMD
// the register allocation is held to.
#ifndef ATTN_BN
#define ATTN_BN 64
#endif
#ifndef ATTN_WAVES_PER_EU
#define ATTN_WAVES_PER_EU 2
#endif

// LDS tile layouts. A K or V tile of BN key rows is BN/4 blocks; block j
// holds rows 4j..4j+3 (4 x 256 bytes) as 64 slots of 16 bytes.
//
// K: the slot of (row 4j + rr, 16-byte chunk c) is rr + 4c, with padding
// between blocks. A ds_read_b128 of 16 lanes covers 4 blocks x 4 rows at
// one chunk: lanes n of the four-wave kernel (rows n of 32) and lanes l%16
// of a 16-lane group of the eight-wave kernel (rows 16kb + l%16). The
// padding of each kernel was chosen by measurement, as the one that shows
// no LDS bank conflicts (SQ_LDS_BANK_CONFLICT = 0) for its read pattern:
// 64 bytes (1088-byte blocks) for the four-wave kernel, 128 bytes (1152)
// for the eight-wave one. With 64 bytes the eight-wave pattern conflicts
// 2-way on every read, and with 128 bytes the four-wave one conflicts too.
// (If a bank were simply (address / 4) % 64, 64 bytes would suit both.)
constexpr int kKBlock = 1088;      // four-wave kernel
constexpr int kKBlockPair = 1152;  // eight-wave kernel
// V: the slot of (row 4j + q, chunk 4b + x) is 16b + 4q + x, blocks 1056
// bytes apart (32 bytes of padding). A transposed read (ds_read_b64_tr_b16)
// is served 32 lanes at a time, 256 bytes over the 64 banks; each 16-lane
// group reads 32 bytes from each of the 4 rows of one block (8 banks per
// row, rows 64 bytes apart). In the four-wave kernel the two groups of a
// half-wave read the two 16-column halves of the same rows; in the
// eight-wave kernel they read the same columns of consecutive blocks, which
// the padding shifts by 8 banks. Either way the 32 lanes meet every bank
// once.
constexpr int kVBlock = 1056;

// Global byte offset (within a 4-row block) that lane l fetches so that its
// 16 bytes land in slot l.
__device__ __forceinline__ int k_fill_offset(int l) {
  const int rr = l & 3, h = (l >> 2) & 1, kk = l >> 3;
  return rr * 256 + (2 * kk + h) * 16;
}
__device__ __forceinline__ int v_fill_offset(int l) {
  const int b = l >> 4, q = (l >> 2) & 3, x = l & 3;
  return q * 256 + (4 * b + x) * 16;
}

template <int BN>
struct Tiles {
  static constexpr int kBlocks = BN / 4;
  static constexpr int kKBytes = kBlocks * kKBlock;
  static constexpr int kVBytes = kBlocks * kVBlock;
  static constexpr int kLoadsPerWave = kBlocks / 4;  // 4 waves share a tile's blocks
};

// Direct-to-LDS loads of one tile: wave w issues blocks w, w+4, w+8, ...
// `g` is the tile's global base (uniform), `lane_off` the lane's fill offset.
template <int BN, int kBlockBytes>
__device__ __forceinline__ void load_tile(const char* g, int lane_off, char* lds, int wave) {
#pragma unroll
  for (int i = 0; i < Tiles<BN>::kLoadsPerWave; ++i) {
    const int j = 4 * i + wave;
    __builtin_amdgcn_global_load_lds(g + j * 1024 + lane_off, (lds_void*)(lds + j * kBlockBytes), 16, 0, 0);
  }
}

// S^T = K . Q^T for one K tile; s[cb] holds keys 32cb + 8j + 4h + i.
template <int BN>
__device__ __forceinline__ void qk_tile(const char* ksm, int k_lane, const bf16x8 (&qf)[8],
                                        f32x16 (&s)[BN / 32]) {
#pragma unroll
  for (int cb = 0; cb < BN / 32; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[cb][i] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ksm + k_lane + cb * 8 * kKBlock + kk * 128);
      s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[cb], 0, 0, 0);
    }
  }
}

// P = 2^(s*c - kept), rounded to bf16, as the PV B operand: step t's
// operand takes slots 0..3 from score block t/2, j = 2(t%2), and slots 4..7
// from j = 2(t%2)+1 (keys 16t + 4h + 0..3 and 16t + 8 + 4h + 0..3). The row
// sum is taken from these rounded values on the matrix pipe (make_selector),
// so O is normalised by exactly the weights its P.V used: the output is a
// convex combination of V rows (normalising by the unrounded sum leaves a
// bias when a few large P round the same way).
// Software 2^x (the article's Chapter 9 idea: compute part of the
// exponentials on the FMA pipe instead of the exponent unit), written from
// 2^x = 2^n * 2^f with n = floor(x), f = x - n in [0, 1) and 2^f by a
// degree-3 polynomial in f. The coefficients minimise the maximum relative
// error on [0, 1] (Remez exchange, with c0 pinned to 1 so integer arguments
// are exact): 8.6e-5 with these float32 values, far below the 2^-9 of the
// bf16 rounding that follows. They are produced by exp2_poly_fit.py beside
// this file. The argument is clamped to [-127, 128] before it is split (one
// v_med3), so every argument below -126 (any finite one, however large)
// gives at most 2^-126, where the exponent unit gives 0, and every one from
// 128 up, +Inf included, gives Inf. The P that the kernel keeps has
// arguments below 1; the larger ones met before a rebase give at least 2 or
// Inf, which set the exponent bit the rebase test reads.
constexpr float kExp2C0 = 1.0f;
constexpr float kExp2C1 = 0.6951163411140442f;
constexpr float kExp2C2 = 0.22764700651168823f;
constexpr float kExp2C3 = 0.07706519961357117f;
__device__ __forceinline__ float exp2_poly(float x) {
  const float xc = __builtin_amdgcn_fmed3f(x, -127.0f, 128.0f);
  const float n = __builtin_floorf(xc);
  const float f = xc - n;
  float p = __builtin_fmaf(kExp2C3, f, kExp2C2);
  p = __builtin_fmaf(p, f, kExp2C1);
  p = __builtin_fmaf(p, f, kExp2C0);
  return __builtin_ldexpf(p, int(n));
}

template <int BN>
__device__ __forceinline__ void exp_tile_p(const f32x16 (&s)[BN / 32], float c, float kept,
                                           bf16x8 (&pf)[BN / 16]) {
#pragma unroll
  for (int cb = 0; cb < BN / 32; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pf[2 * cb + (j >> 1)][(j & 1) * 4 + i] =
            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][4 * j + i], c, -kept));
}

// The other half-wave's value of x (lane l <-> lane l ^ 32), through
// v_permlane32_swap, which exchanges the upper half of its first operand
// with the lower half of its second: with x in both, lanes 0-31 find the
// partner's value in the second result and lanes 32-63 in the first.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Raw row max of a score tile over both half-waves, with v_maximum3 (fmaxf's
// NaN rule would add a quieting v_max per MFMA result; inputs are finite
// by contract) and the half-wave exchange on v_permlane32_swap.
template <int BN>
__device__ __forceinline__ float tile_max_swap(const f32x16 (&s)[BN / 32]) {
  // Two running maxima, each taking two values per v_maximum3_f32: 33
  // instructions for a lane's 2 * BN scores, on chains half as long.
  float m0 = __builtin_elementwise_maximum(s[0][0], s[0][1]);
  float m1 = __builtin_elementwise_maximum(s[0][2], s[0][3]);
#pragma unroll
  for (int cb = 0; cb < BN / 32; ++cb)
#pragma unroll
    for (int i = cb == 0 ? 4 : 0; i < 16; i += 4) {
      m0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m0, s[cb][i]), s[cb][i + 1]);
      m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m1, s[cb][i + 2]), s[cb][i + 3]);
    }
  return max_with_other_half(__builtin_elementwise_maximum(m0, m1));
}

// A operand of the row-sum MFMA. v_mfma_f32_16x16x32_bf16 takes a PV
// fragment as its B operand: lane l holds 8 keys of query l % 32, in the
// 16x16x32 layout column l % 16 and k-group l / 16 (groups 0 and 2 belong to
// query c = l % 16, groups 1 and 3 to query c + 16). Selector row r has ones
// on the groups of query c (r = 0, 8) or c + 16 (r = 4, 12) and zeros
// elsewhere; output row 4 * (l / 16) of column l % 16 then lands in lane l,
// register 0, as the sum over the step's 16 keys for query l % 32.
// Registers 1-3 of the accumulator stay 0.
__device__ __forceinline__ bf16x8 make_selector(int lane) {
  const int r = lane & 15, g = lane >> 4;
  const bool on = ((r == 0 || r == 8) && !(g & 1)) || ((r == 4 || r == 12) && (g & 1));
  bf16x8 sel;
#pragma unroll
  for (int e = 0; e < 8; ++e) sel[e] = (__bf16)(on ? 1.0f : 0.0f);
  return sel;
}

// O^T[d-block b] += V^T[b, step t] . P^T[step t] for one V tile.
template <int BN>
__device__ __forceinline__ void pv_tile(const char* vsm, int v_lane, const bf16x8 (&pf)[BN / 16],
                                        f32x16 (&acc)[4], f32x4& lacc, const bf16x8& sel) {
#pragma unroll
  for (int t = 0; t < BN / 16; ++t) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const char* p0 = vsm + v_lane + t * 4 * kVBlock + b * 256;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(p0 + 2 * kVBlock));
      const i16x8 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16), pf[t],
                                                       acc[b], 0, 0, 0);
    }
    // the row sum of the same rounded P (see make_selector)
    lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pf[t], lacc, 0, 0, 0);
  }
}

// Online-softmax base update for a new tile max (raw units): rebase when
// the scaled max exceeds the kept base by >= kRebaseLog2, rescaling O and the row sum
// only if some lane of the wave rebased.
__device__ __forceinline__ void update_base(float raw_max, float c, float& kept, f32x4& lacc,
                                            f32x16 (&acc)[4]) {
  const float cand = __builtin_elementwise_maximum(kept, raw_max * c);
  const bool need = (cand - kept) >= kRebaseLog2;
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(kept - cand) : 1.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;
    lacc[0] *= alpha;
    kept = need ? cand : kept;
  }
}

// One K/V-loop iteration. On entry S(jt) is in `s` with its base applied,
// K(jt+1) is in `k_next` and V(jt) in `v_cur`; S(jt+1) is left in `sn`. Loads of K(jt+2) (into
// `k_cur`, freed at the previous barrier) and V(jt+1) (into `v_next`) are
// issued first and land during the iteration.
template <int BN>
__device__ __forceinline__ void kv_iteration(int jt, int ntiles, const char* kg, const char* vg,
                                             int kfill, int vfill, int wave, char* k_cur,
                                             char* k_next, char* v_cur, char* v_next, int k_lane,
                                             int v_lane, const bf16x8 (&qf)[8], float c,
                                             const f32x16 (&s)[BN / 32], f32x16 (&sn)[BN / 32],
                                             f32x16 (&acc)[4], float& kept, f32x4& lacc,
                                             const bf16x8& sel) {
  constexpr int kTileBytes = BN * kD * 2;
  if (jt + 2 < ntiles) load_tile<BN, kKBlock>(kg + int64_t(jt + 2) * kTileBytes, kfill, k_cur, wave);
  if (jt + 1 < ntiles) load_tile<BN, kVBlock>(vg + int64_t(jt + 1) * kTileBytes, vfill, v_next, wave);

  bf16x8 pf[BN / 16];
  exp_tile_p<BN>(s, c, kept, pf);
  // QK^T of the next tile, issued without a branch so it can interleave
  // with the exponentials above; on the last tile it reads a stale (but
  // in-bounds) buffer and its result is dropped.
  qk_tile<BN>(k_next, k_lane, qf, sn);
  pv_tile<BN>(v_cur, v_lane, pf, acc, lacc, sel);
  if (jt + 1 < ntiles) update_base(tile_max_swap<BN>(sn), c, kept, lacc, acc);
  __syncthreads();  // K(jt+2), V(jt+1) landed; K(jt+1), V(jt) are free
}

template <int BN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ATTN_WAVES_PER_EU, ATTN_WAVES_PER_EU)))
void attn_fwd_kernel(const uint4* __restrict__ q, const char* __restrict__ k,
                     const char* __restrict__ v, __bf16* __restrict__ o, float* __restrict__ lse,
                     int S, int qtiles, int nwg, float c) {
  static_assert(BN % 64 == 0, "tile shape: 4 waves x 4-row blocks, 32-key score blocks");
  constexpr int kTileBytes = BN * kD * 2;
  using T = Tiles<BN>;
  // K and V each have two buffers, as separate objects so that reads of
  // one need not wait for direct-to-LDS loads into the other.
  __shared__ uint4 k0[T::kKBytes / 16], k1[T::kKBytes / 16];
  __shared__ uint4 v0[T::kVBytes / 16], v1[T::kVBytes / 16];
  char* const kb0 = reinterpret_cast<char*>(k0);
  char* const kb1 = reinterpret_cast<char*>(k1);
  char* const vb0 = reinterpret_cast<char*>(v0);
  char* const vb1 = reinterpret_cast<char*>(v1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // query column within the wave's 32 rows
  const int h = lane >> 5;   // half-wave

  // XCD-aware renumbering: block i runs on XCD i % 8; give XCD x the
  // contiguous work range [x*per, (x+1)*per).
  const int bid = blockIdx.x;
  const int per = nwg >> 3;
  const int work = bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bh = work / qtiles;
  const int qt = work - bh * qtiles;
  const int64_t head = int64_t(bh) * S * kD;  // element offset of this (b, h)

  const char* kg = k + head * 2;
  const char* vg = v + head * 2;
  const int ntiles = S / BN;
  const int kfill = k_fill_offset(lane);
  const int vfill = v_fill_offset(lane);

  // Per-lane LDS read bases (see the layout notes).
  const int k_lane = (n >> 2) * kKBlock + ((n & 3) + 4 * h) * 16;
  const int v_lane = h * kVBlock + 64 * ((lane & 15) >> 2) +
                     16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);

  // Prologue loads: K0, V0 and K1.
  load_tile<BN, kKBlock>(kg, kfill, kb0, wave);
  load_tile<BN, kVBlock>(vg, vfill, vb0, wave);
  if (ntiles > 1) load_tile<BN, kKBlock>(kg + kTileBytes, kfill, kb1, wave);

  // Q fragments (B operand of S^T = K Q^T): lane holds its query's
  // dims 16kk + 8h .. +7 for kk = 0..7, loaded once.
  const int qrow = qt * kBM + wave * 32 + n;
  const uint4* qp = q + ((head + int64_t(qrow) * kD) >> 3);
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, qp[2 * kk + h]);

  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.0f;
  float kept = -FLT_MAX;  // kept row max, base-2 units of scaled scores
  f32x4 lacc = {0.0f, 0.0f, 0.0f, 0.0f};  // row sum in register 0 (see make_selector)
  const bf16x8 sel = make_selector(lane);

  f32x16 s0[BN / 32], s1[BN / 32];
  __syncthreads();  // K0, V0 (and K1) are in LDS
  qk_tile<BN>(kb0, k_lane, qf, s0);
  update_base(tile_max_swap<BN>(s0), c, kept, lacc, acc);
  __syncthreads();  // everyone is done reading K0

  // Iterations alternate the roles of the two K buffers, the two V buffers
  // and the two score register sets.
  for (int jt = 0; jt < ntiles; jt += 2) {
    kv_iteration<BN>(jt, ntiles, kg, vg, kfill, vfill, wave, kb0, kb1, vb0, vb1, k_lane, v_lane, qf,
                     c, s0, s1, acc, kept, lacc, sel);
    if (jt + 1 >= ntiles) break;
    kv_iteration<BN>(jt + 1, ntiles, kg, vg, kfill, vfill, wave, kb1, kb0, vb1, vb0, k_lane, v_lane,
                     qf, c, s1, s0, acc, kept, lacc, sel);
  }

  // Epilogue: O = O^T / l -> bf16; lane holds dims 32b + 8j + 4h + 0..3.
  const float ltot = lacc[0];
  const float inv = 1.0f / ltot;
  __bf16* orow = o + head + int64_t(qrow) * kD;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc[b][4 * j + i] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * j + 4 * h) = w;
    }
  if (h == 0) lse[int64_t(bh) * S + qrow] = (kept + __log2f(ltot)) * kLn2;
}

// Waits until this wave's direct-to-LDS loads and LDS reads have completed
// (s_waitcnt vmcnt(0) lgkmcnt(0)); the data is then visible to the whole
// workgroup after the next barrier.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0x0070); }
// s_waitcnt vmcnt(0) alone: this wave's loads have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for loads that are meant to stay in flight across it). The
// scheduling barriers stop the compiler from moving arithmetic across it,
// which would blur the phases the barrier separates.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// MFMA-phase settings per query-block count QB: LDS operand fragments in
// flight and fragments that share one s_waitcnt. (With either QB the wave
// also raises its issue priority for the phase; see the kernel loop.)
//  * QB = 2: a wave waits for 4 fragments' reads at once, so 48 of the
//    phase's 64 waits go away (every instruction a wave issues between its
//    MFMAs delays the next one), with 6 in flight to keep 2 fragments' reads
//    ahead of the group awaited. With the priority: +1-4% at 16K keys,
//    +0-0.6% at 4K and 8K.
//  * QB = 1: one wait per fragment and 4 in flight: its phase is bound by
//    LDS reads (each fragment feeds one MFMA), and grouped waits with 6 in
//    flight measured slower there.
template <int QB>
struct MmaCfg {
  static constexpr int kPrefetch = QB == 2 ? 6 : 4;
  static constexpr int kWaitGroup = QB == 2 ? 4 : 1;
};

// LDS reads of the MFMA phase are issued as inline assembly with explicit
// s_waitcnt lgkmcnt(N): the compiler's own counting gives up (waits for
// everything) as soon as the loop also holds direct-to-LDS loads, which
// would drain the operand ring every few MFMAs. LDS reads of one wave
// complete in issue order, so N = the number of reads issued after the last
// one awaited. A scheduling barrier after each wait keeps every use of the
// awaited registers below it (naming them as in/out operands of the wait
// did too, but made the hazard recognizer pad each MFMA with an s_nop);
// volatile asm statements keep their order among themselves.
template <int kOff>
__device__ __forceinline__ u32x4 lds_b128(unsigned addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff));
  return r;
}
template <int kOff0, int kOff1>
__device__ __forceinline__ void lds_tr_pair(unsigned addr, u32x2& lo, u32x2& hi) {
  // Early-clobber outputs: the second read takes its address after the
  // first has been issued, so `lo` must not be given the address register
  // (the first read may land before the second issues when the LDS queue
  // is full).
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(lo), "=&v"(hi) : "v"(addr), "i"(kOff0), "i"(kOff1));
}
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" :: "i"(N));
  __builtin_amdgcn_sched_barrier(0);
}

// Ring of LDS operand fragments of an MFMA phase, PF deep.
template <int PF>
struct MmaRing {
  u32x4 k[PF];
  u32x2 vlo[PF], vhi[PF];
};

// ---------------------------------------------------------------------------
// Eight-wave kernel (variants PAIR256, PAIR256_EXP2EMU, PAIR128) on
// v_mfma_f32_16x16x32_bf16. Same LDS layouts and tile loads as the four-wave
// kernel; a stream of 16x16x32 MFMAs sustains a markedly higher rate on
// gfx950 than one of 32x32x16 MFMAs, though both do 1024 FLOPs per cycle
// per SIMD on paper (about 1.95 against 1.55-1.77 PFLOP/s on N(0,1) bf16
// operands, the lower figure with two waves interleaving MFMAs on a SIMD).
//
// D[16x16] += A[16x32] . B[32x16]: lane l holds row l%16 of A and column
// l%16 of B, each with k = 8g .. 8g+7 where g = l/16, and column l%16 of D
// at rows 4g .. 4g+3. Each wave owns QB 16-query blocks qb: QB = 2 (32
// queries, 128-row tiles per group; PAIR256) or QB = 1 (16 queries, 64-row
// tiles; PAIR128, for grids too small to fill the GPU otherwise).
//  * S^T = K . Q^T per 16-key block kb: A = K rows (keys) from LDS, B = Q
//    (registers). Lane l then holds query 16qb + l%16, keys 16kb + 4g + i.
//    A query's scores are spread over the four lane groups g, so the row
//    max ends with two exchanges (v_permlane16_swap, v_permlane32_swap).
//  * O^T += V^T . P^T per 32-key step t and 16-column block db of d. The k
//    slot 8g + j of both operands stands for key 32t + 4g + j (j < 4) or
//    32t + 16 + 4g + (j - 4) (j >= 4): exactly the keys the lane's two
//    score blocks 2t and 2t+1 hold, so P needs no data movement. V^T is
//    gathered for those keys with two ds_read_b64_tr_b16 per fragment.
//  * The row sum takes one v_smfmac_f32_16x16x64_bf16 per two steps: the B
//    operand is the two steps' P side by side (64 keys), the sparse A is all
//    ones and keeps, of each group of four k slots, slots {0, 1} in rows
//    0-7 and {2, 3} in rows 8-15. Rows 0-7 of D (lanes 0-31) and rows 8-15
//    (lanes 32-63) thus hold complementary halves of lane l's key sum,
//    added once at the end. Half the matrix-pipe slots of a dense all-ones
//    16x16x32 per step, at the same issue rate (17.1 ticks either way in a
//    microbenchmark). The MFMA wave issues those of P(i-1) at the start of
//    its phase, right after its first fragments' reads, whose latency they
//    fill (the softmax phase before has already applied its factor alpha to
//    the sums).
//  * With QB = 2 every K and V fragment read from LDS feeds the MFMAs of
//    both query blocks, so LDS traffic per FLOP is that of the four-wave
//    kernel's 32x32x16 MFMAs (one fragment per 32x32 output block). With
//    QB = 1 it doubles, and so do the LDS instructions a wave issues per
//    MFMA. With QB = 2 the refill of a ring slot (fragment F + PF) is split
//    around fragment F's two MFMAs: MFMA, read, MFMA, read (the one read of
//    a K fragment goes between them). One LDS instruction between MFMAs
//    costs a wave less than two back to back: in a microbenchmark of 4
//    MFMA waves beside softmax waves PV fell from 19.45 to 18.61 ticks per
//    MFMA, QK from 18.30 to 18.14. Issuing a wait group's MFMAs query block
//    by query block, with the group's refills after all eight, measured 10%
//    slower.
// ---------------------------------------------------------------------------

// Fragments of an MFMA phase in issue order: first the V fragments of
// PV(i-1) (step t, d block db), then the K fragments of QK(i) (score block
// kb, 32-dim step). PV first lets the P operands die before the scores are
// written, which keeps the phase within the register budget.
template <int BN>
struct Frags16 {
  static constexpr int kKB = BN / 16;       // 16-key score blocks per tile
  static constexpr int kV = BN / 4;         // V fragments: BN/32 steps x 8 d blocks
  static constexpr int kTotal = kV + kKB * 4;
  static constexpr int ops(int f) { return f < kV ? 2 : 1; }
  // LDS reads that may still be in flight when fragments f .. f + wg - 1
  // must have landed, with fragments up to f + pf - 1 issued.
  static constexpr int after(int f, int pf, int wg, int end = kTotal) {
    int n = 0;
    for (int g = f + wg; g < f + pf && g < end; ++g) n += ops(g);
    return n;
  }
  // Fragments awaited together ("wait groups") with a group size of wg:
  // {0}, {1}, {2, 3}, then wg at a time from fragment wg on, so the phase's
  // first MFMAs start as soon as their own fragment has landed (+0.2-0.7%
  // against groups of 4 from the start). With wg = 1 every fragment waits.
  static constexpr bool group_start(int f, int wg) { return wg == 1 || f <= 2 || f % wg == 0; }
  static constexpr int group_len(int f, int wg) { return wg == 1 || f < 2 ? 1 : f == 2 ? 2 : wg; }
};

template <int BN, int PF, int F>
__device__ __forceinline__ void issue_frag16(MmaRing<PF>& ring, unsigned kaddr, unsigned vaddr) {
  constexpr int slot = F % PF;
  if constexpr (F < Frags16<BN>::kV) {
    constexpr int db = F % 8, t = F / 8;
    constexpr int off = t * 8 * kVBlock + 256 * (db >> 1) + 32 * (db & 1);
    lds_tr_pair<off, off + 4 * kVBlock>(vaddr, ring.vlo[slot], ring.vhi[slot]);
  } else {
    constexpr int f = F - Frags16<BN>::kV;
    constexpr int kb = f % Frags16<BN>::kKB, step = f / Frags16<BN>::kKB;
    ring.k[slot] = lds_b128<kb * 4 * kKBlockPair + step * 256>(kaddr);
  }
}

// Half of the refill of fragment F: part 0 is the first transposing read of
// a V fragment or the one read of a K fragment, part 1 the second
// transposing read (nothing for a K fragment).
template <int BN, int PF, int F, int kPart>
__device__ __forceinline__ void issue_half16(MmaRing<PF>& ring, unsigned kaddr, unsigned vaddr) {
  constexpr int slot = F % PF;
  if constexpr (F < Frags16<BN>::kV) {
    constexpr int db = F % 8, t = F / 8;
    constexpr int off = t * 8 * kVBlock + 256 * (db >> 1) + 32 * (db & 1) + kPart * 4 * kVBlock;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(kPart == 0 ? ring.vlo[slot] : ring.vhi[slot]) : "v"(vaddr), "i"(off));
  } else if constexpr (kPart == 0) {
    constexpr int f = F - Frags16<BN>::kV;
    constexpr int kb = f % Frags16<BN>::kKB, step = f / Frags16<BN>::kKB;
    ring.k[slot] = lds_b128<kb * 4 * kKBlockPair + step * 256>(kaddr);
  }
}

template <int BN, int QB, int F, int kEnd = Frags16<BN>::kTotal>
__device__ __forceinline__ void mma_step16(MmaRing<MmaCfg<QB>::kPrefetch>& ring, unsigned kaddr, unsigned vaddr,
                                           const bf16x8 (&qf)[QB][4], f32x4 (&s)[BN / 16][QB],
                                           const bf16x8 (&pf)[QB][BN / 32], f32x4 (&acc)[8][QB]) {
  constexpr int PF = MmaCfg<QB>::kPrefetch, WG = MmaCfg<QB>::kWaitGroup;
  static_assert(kEnd % WG == 0 && WG < PF && (WG == 1 || WG == 4),
                "fragments are awaited in whole groups, with reads of later ones in flight");
  constexpr int slot = F % PF;
  constexpr bool kSplit = QB == 2 && F + PF < kEnd;
  // the first fragment of a wait group waits for all of the group
  constexpr bool wait = Frags16<BN>::group_start(F, WG);
  constexpr int N = Frags16<BN>::after(F, PF, Frags16<BN>::group_len(F, WG), kEnd);
  if constexpr (F < Frags16<BN>::kV) {
    constexpr int db = F % 8, t = F / 8;
    if constexpr (wait) lgkm_wait<N>();
    const u32x4 a = __builtin_shufflevector(ring.vlo[slot], ring.vhi[slot], 0, 1, 2, 3);
    // In place through tied operands: each O accumulator keeps one register
    // set (with the builtin the allocator moved the accumulators between
    // two sets every phase).
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[db][0]) : "v"(a), "v"(pf[0][t]));
    if constexpr (QB == 2) {
      if constexpr (kSplit) issue_half16<BN, PF, F + PF, 0>(ring, kaddr, vaddr);
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[db][QB - 1]) : "v"(a), "v"(pf[QB - 1][t]));
      if constexpr (kSplit) issue_half16<BN, PF, F + PF, 1>(ring, kaddr, vaddr);
    }
  } else {
    constexpr int f = F - Frags16<BN>::kV;
    constexpr int kb = f % Frags16<BN>::kKB, step = f / Frags16<BN>::kKB;
    if constexpr (wait) lgkm_wait<N>();
    const bf16x8 a = __builtin_bit_cast(bf16x8, ring.k[slot]);
    const f32x4 zero = {};
    s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][step], step == 0 ? zero : s[kb][0], 0, 0, 0);
    if constexpr (kSplit) {
      __builtin_amdgcn_sched_barrier(0);
      issue_half16<BN, PF, F + PF, 0>(ring, kaddr, vaddr);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (QB == 2)
      s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][step], step == 0 ? zero : s[kb][1], 0, 0, 0);
    if constexpr (kSplit) issue_half16<BN, PF, F + PF, 1>(ring, kaddr, vaddr);
  }
  if constexpr (!kSplit && F + PF < kEnd) issue_frag16<BN, PF, F + PF>(ring, kaddr, vaddr);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (F + 1 < kEnd)
    mma_step16<BN, QB, F + 1, kEnd>(ring, kaddr, vaddr, qf, s, pf, acc);
}

template <int BN, int PF, int F>
__device__ __forceinline__ void issue_first16(MmaRing<PF>& ring, unsigned kaddr, unsigned vaddr) {
  issue_frag16<BN, PF, F>(ring, kaddr, vaddr);
  if constexpr (F + 1 < PF) issue_first16<BN, PF, F + 1>(ring, kaddr, vaddr);
}

// MFMA phase i >= 1: the O rescale chosen by softmax phase i-1 (only if
// some row of the wave rebased; that phase already rescaled the row sums),
// the row sums of P(i-1) while the first fragments' reads are in flight,
// PV(i-1) and QK(i), then publish this wave's finished loads and pass a
// barrier (unless `nobarrier`: group B's last phase, which no phase of
// group A waits for). The next rescale reads O long after its last MFMA
// (the QK steps follow it). With kEnd = the V fragment count the phase
// stops after PV: the last phase, which has no tile to score (the epilogue
// reads O after its wait for the reads, long after the MFMAs issued).
template <int BN, int QB, int kEnd = Frags16<BN>::kTotal>
__device__ __forceinline__ void pp_m_phase(const char* ksm, const char* vsm, int k_lane, int v_lane,
                                             const bf16x8 (&qf)[QB][4], f32x4 (&s)[BN / 16][QB],
                                             const bf16x8 (&pf)[QB][BN / 32], f32x4 (&acc)[8][QB],
                                             const float (&alpha)[QB], bool rescale, bool nobarrier,
                                             f32x4 (&lacc)[QB], const bf16x8& ones, int sidx) {
  if (rescale) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db][qb] *= alpha[qb];
    }
    // The PV MFMAs below are inline assembly, which the compiler's hazard
    // checks do not see: give the VALU writes their wait states here.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      asm volatile("s_nop 4" : "+v"(acc[0][qb]), "+v"(acc[1][qb]), "+v"(acc[2][qb]), "+v"(acc[3][qb]),
                   "+v"(acc[4][qb]), "+v"(acc[5][qb]), "+v"(acc[6][qb]), "+v"(acc[7][qb]));
  }
  const unsigned kaddr = unsigned(reinterpret_cast<uintptr_t>(ksm)) + unsigned(k_lane);
  const unsigned vaddr = unsigned(reinterpret_cast<uintptr_t>(vsm)) + unsigned(v_lane);
  MmaRing<MmaCfg<QB>::kPrefetch> ring;
  issue_first16<BN, MmaCfg<QB>::kPrefetch, 0>(ring, kaddr, vaddr);
  __builtin_amdgcn_sched_barrier(0);
  // The row sums of P(i-1) while the first fragments' reads are in flight.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < BN / 32; t += 2) {
      const bf16x16 b = __builtin_shufflevector(pf[qb][t], pf[qb][t + 1], 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                                12, 13, 14, 15);
      lacc[qb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(ones, b, lacc[qb], sidx, 0, 0);
    }
  __builtin_amdgcn_sched_barrier(0);
  mma_step16<BN, QB, 0, kEnd>(ring, kaddr, vaddr, qf, s, pf, acc);
  if constexpr (kEnd != Frags16<BN>::kTotal) {
    // The epilogue's VALU instructions read O next, and the compiler's
    // hazard checks do not see the MFMAs above (inline assembly): wait out
    // an 8-pass MFMA's result latency (11 wait states) here.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      asm volatile("s_nop 7\n\ts_nop 3" : "+v"(acc[0][qb]), "+v"(acc[1][qb]), "+v"(acc[2][qb]), "+v"(acc[3][qb]),
                   "+v"(acc[4][qb]), "+v"(acc[5][qb]), "+v"(acc[6][qb]), "+v"(acc[7][qb]));
  }
  wait_mem();
  if (nobarrier) return;
  barrier();
}

// QK of the first K tile alone, with plain builtins.
template <int BN, int QB>
__device__ __forceinline__ void qk16_tile(const char* ksm, int k_lane, const bf16x8 (&qf)[QB][4],
                                          f32x4 (&s)[BN / 16][QB]) {
#pragma unroll
  for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8*>(ksm + k_lane + kb * 4 * kKBlockPair + step * 256);
      const f32x4 zero = {};
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qb][step], step == 0 ? zero : s[kb][qb],
                                                            0, 0, 0);
    }
}

// Max of x over the four lanes l%16 + 16g that hold one query's scores.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The same for two values at once (the row maxima of two query blocks):
// the first exchange pairs x0's and x1's lane groups in one swap, which
// leaves x0's partial maxima in groups 0 and 2 and x1's in groups 1 and 3;
// after the 32-lane exchange the last 16-lane swap hands out both results
// without a further maximum. Seven instructions instead of twelve.
__device__ __forceinline__ void max_over_groups2(float x0, float x1, float& y0, float& y1) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const float y = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  const float z = __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  y0 = __uint_as_float(c[0]);
  y1 = __uint_as_float(c[1]);
}

// Raw row max of query block qb over the lane's 4 * BN/16 scores (two
// v_maximum3 chains), before the exchange between lane groups.
template <int BN, int QB>
__device__ __forceinline__ float lane_max16(const f32x4 (&s)[BN / 16][QB], int qb) {
  float m0 = __builtin_elementwise_maximum(s[0][qb][0], s[0][qb][1]);
  float m1 = __builtin_elementwise_maximum(s[0][qb][2], s[0][qb][3]);
#pragma unroll
  for (int kb = 1; kb < BN / 16; ++kb) {
    m0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m0, s[kb][qb][0]), s[kb][qb][1]);
    m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m1, s[kb][qb][2]), s[kb][qb][3]);
  }
  return __builtin_elementwise_maximum(m0, m1);
}

// Raw row maxima of the wave's query blocks over the tile.
template <int BN, int QB>
__device__ __forceinline__ void tile_max16(const f32x4 (&s)[BN / 16][QB], float (&raw)[QB]) {
  if constexpr (QB == 2)
    max_over_groups2(lane_max16<BN, QB>(s, 0), lane_max16<BN, QB>(s, 1), raw[0], raw[1]);
  else
    raw[0] = max_over_groups(lane_max16<BN, QB>(s, 0));
}

// P = 2^(s*c - kept) in bf16 as PV B operands, for score blocks kb0 .. kb1-1
// of query block qb: step t takes slots 0..3 from score block 2t and slots
// 4..7 from block 2t+1. kEmuEvery = 0: every exponential on v_exp_f32.
// kEmuEvery = k: one element in k (those with (4 kb + i) % k == k - 1) takes
// exp2_poly instead.
template <int BN, int QB, int kEmuEvery, int qb, int kb0, int kb1>
__device__ __forceinline__ void exp16_part(const f32x4 (&s)[BN / 16][QB], float c, const float (&kept)[QB],
                                           bf16x8 (&pf)[QB][BN / 32]) {
#pragma unroll
  for (int kb = kb0; kb < kb1; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = __builtin_fmaf(s[kb][qb][i], c, -kept[qb]);
      const bool emu = kEmuEvery > 0 && (4 * kb + i) % (kEmuEvery > 0 ? kEmuEvery : 1) == kEmuEvery - 1;
      pf[qb][kb >> 1][(kb & 1) * 4 + i] = (__bf16)(emu ? exp2_poly(x) : __builtin_amdgcn_exp2f(x));
    }
}

// Softmax phase i: this group's share of the tile loads (below), spread
// over P(i), the rebase test on P(i) (with the row max, the base update and
// its factor alpha only when it fires; the next MFMA phase applies alpha to
// O, which already holds PV(i-1)), and alpha applied to the row sums, which
// hold P up to P(i-1) (the next MFMA phase adds those of P(i)).
template <int BN, int QB, int kEmuEvery, bool kFirst>
__device__ __forceinline__ void pp_v_phase(int i, int group, int wave,
                                             const char* lsrc, int ntiles, int fill, char* kfree,
                                             char* vcur, float c, const f32x4 (&s)[BN / 16][QB],
                                             bf16x8 (&pf)[QB][BN / 32], float (&alpha)[QB],
                                             bool& rescale, float (&kept)[QB], f32x4 (&lacc)[QB],
                                             const bf16x8& ones, int sidx) {
  constexpr int kTileBytes = BN * kD * 2;
  static_assert(Tiles<BN>::kLoadsPerWave == 8 && BN / 16 == 8, "load spread assumes 128-key tiles");
  // The two groups split the loads so that each phase pair moves one tile:
  // group B fetches K(i+2) into the buffer K(i) left, group A fetches V(i)
  // into the buffer V(i-2) left (both buffers' last readers finished in the
  // previous interval). A waits for its loads at the end of this phase;
  // B's are awaited at the end of its next MFMA phase.
  //
  // The 4 waves of a group move 32 KB per phase through the CU's vector
  // memory path, and a wave's load issue stalls while that path is busy.
  // The wave's 8 loads are therefore spread over the phase instead of being
  // issued up front: two at its start, two after the first query block's
  // exponentials and four after half of the second's. (When the phase began
  // with the row max, starting the loads before it was 1-1.5% slower at 4K
  // and 8K keys; with the exponentials first, other spreads measured the
  // same.)
  //
  // The loads go through a raw buffer resource over the one tile they
  // fetch (of K for group B, of V for group A, from `lsrc`), so that the
  // block offsets stay in scalar registers and the lane's byte offset
  // `fill` is fixed. They are issued in every phase: group B's last two
  // (K tiles ntiles and ntiles + 1) get a resource of zero length, so the
  // hardware's range check turns them into zero fills, without a memory
  // access, of a K buffer that no QK reads.
  const bool kside = group == 1;
  const int tile = kside ? i + 2 : i;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(lsrc + int64_t(tile) * kTileBytes), 0, tile < ntiles ? kTileBytes : 0, kBufferWord3);
  char* const dst = kside ? kfree : vcur;
  const int stride = kside ? kKBlockPair : kVBlock;
  auto issue2 = [&](int ii) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = 4 * (ii + x) + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + j * stride), 16, fill, j * 1024, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Exponentials first, against the kept base, which sits kBitRebaseLog2 - 1
  // above the row's max * c at its last rebase: P < 2 for every score below
  // the threshold, so the top exponent bit of a bf16 P (P >= 2) flags a row
  // that must rebase, overflow to Inf included. One OR over P's words tests
  // the whole wave. Only when some row is flagged (a wave-uniform branch,
  // rare after the first tile) are the row max, the new base and the factor
  // alpha computed and P recomputed, so no tile pays for a row max before
  // its exponentials. Otherwise alpha keeps its stale value, which the MFMA
  // phase does not read. The empty assembly statements pin each part of P
  // before the next loads (the compiler would otherwise sink all
  // exponentials below them).
  if constexpr (kFirst) {
    // Every row rebases on its first tile (its base starts at -FLT_MAX), so
    // the first phase goes straight to the row max.
    issue2(0);
    issue2(2);
    issue2(4);
    issue2(6);
    rescale = true;
  } else {
    issue2(0);
    if constexpr (QB == 2) {
      exp16_part<BN, QB, kEmuEvery, 0, 0, 8>(s, c, kept, pf);
      asm volatile("" : "+v"(pf[0][0]), "+v"(pf[0][1]), "+v"(pf[0][2]), "+v"(pf[0][3]));
      issue2(2);
      exp16_part<BN, QB, kEmuEvery, QB - 1, 0, 4>(s, c, kept, pf);
      asm volatile("" : "+v"(pf[QB - 1][0]), "+v"(pf[QB - 1][1]));
      issue2(4);
      issue2(6);
      exp16_part<BN, QB, kEmuEvery, QB - 1, 4, 8>(s, c, kept, pf);
    } else {
      exp16_part<BN, QB, kEmuEvery, 0, 0, 4>(s, c, kept, pf);
      asm volatile("" : "+v"(pf[0][0]), "+v"(pf[0][1]));
      issue2(2);
      exp16_part<BN, QB, kEmuEvery, 0, 4, 6>(s, c, kept, pf);
      asm volatile("" : "+v"(pf[0][2]));
      issue2(4);
      issue2(6);
      exp16_part<BN, QB, kEmuEvery, 0, 6, 8>(s, c, kept, pf);
    }
    unsigned bits = 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int t = 0; t < BN / 32; ++t) {
        const u32x4 w = __builtin_bit_cast(u32x4, pf[qb][t]);
        bits |= w[0] | w[1] | w[2] | w[3];
      }
    rescale = __builtin_amdgcn_ballot_w64((bits & 0x40004000u) != 0u) != 0;
  }
  if (rescale) {
    float raw[QB];
    tile_max16<BN, QB>(s, raw);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m = __builtin_fmaf(raw[qb], c, kBitRebaseLog2 - 1.0f);
      const bool need = m - kept[qb] >= kBitRebaseLog2;
      alpha[qb] = need ? __builtin_amdgcn_exp2f(kept[qb] - m) : 1.0f;
      kept[qb] = need ? m : kept[qb];
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (qb == 0) exp16_part<BN, QB, kEmuEvery, 0, 0, BN / 16>(s, c, kept, pf);
      else exp16_part<BN, QB, kEmuEvery, QB - 1, 0, BN / 16>(s, c, kept, pf);
    }
  }
  // P must be complete here, not computed after the barrier where it is
  // first used: the overlap of this phase with the other group's MFMAs
  // depends on it.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) asm volatile("" : "+v"(pf[qb][t]));
  // The row sums (up to P(i-1)) take the factor of this tile's base update.
  if (rescale) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lacc[qb] *= alpha[qb];
  }
  if (group == 0) wait_vmem();
  barrier();
}

// Eight-wave kernel: two 4-wave groups own two consecutive 128-row Q tiles
// of one head and share every K/V tile (the article's two-Q-tile CTA,
// Chapter 5). Barriers make the groups alternate: while one group runs
// its MFMA phase [PV(i-1), QK(i)] the other runs its softmax phase on the
// SIMD it shares (the role split of Chapters 4 and 12, done here by
// phase-shifting two groups of identical waves instead of specialised warps).
//
// Group A runs M(0) V(0) M(1) V(1) ... M(n), where M(0) is QK(0) alone and
// M(n) PV(n-1) alone; group B starts one barrier later, so interval 2i+1
// holds A's V(i) and B's M(i), interval 2i+2 A's M(i+1) and B's V(i). K(i) and V(i) live in buffer i%2. K(i+2) is loaded
// by group B during its V(i) and awaited at the end of its M(i+1); V(i) is
// loaded by group A during its V(i) and awaited at its end. Each interval
// thus moves one tile through the load path (issuing both in one phase
// stalled that phase for the whole transfer). Before the loop all eight
// waves load K(0) and K(1), and each group its Q tile.
//
// All workgroups of a launch do equal work, so those of one round over the
// CUs start and end together, and the Q reads at a round's start and the O
// writes at its end come as bursts at the memory's bandwidth. Hence the
// first barrier waits only for what group A's QK(0) needs (K(0) and A's Q),
// and at the end group A stores its rows during group B's last MFMA phase,
// which ends without a barrier (group A passes none after its own last
// phase, so the counts match).
//
// The softmax phase computes P against the kept base and tests it for a
// rebase (the row max and the base update run only when that test fires);
// the MFMA phase issues the previous P's row sums (in the shadow of its
// first reads) and the MFMAs of PV and QK with their LDS reads.
template <int BN, int QB, int kEmuEvery>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pingpong_kernel(const uint4* __restrict__ q, const char* __restrict__ k,
                          const char* __restrict__ v, __bf16* __restrict__ o,
                          float* __restrict__ lse, int S, int qtiles, int npairs, int nwg, float c) {
  static_assert(BN % 64 == 0, "tile shape");
  constexpr int kTileBytes = BN * kD * 2;
  using T = Tiles<BN>;
  __shared__ uint4 k0[T::kBlocks * kKBlockPair / 16], k1[T::kBlocks * kKBlockPair / 16];
  __shared__ uint4 v0[T::kVBytes / 16], v1[T::kVBytes / 16];
  char* const kb0 = reinterpret_cast<char*>(k0);
  char* const kb1 = reinterpret_cast<char*>(k1);
  char* const vb0 = reinterpret_cast<char*>(v0);
  char* const vb1 = reinterpret_cast<char*>(v1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave8 >> 2;
  const int wave = wave8 & 3;
  const int col = lane & 15;  // query within a 16-query block
  const int g = lane >> 4;    // lane group

  const int bid = blockIdx.x;
  const int per = nwg >> 3;
  const int work = bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bh = work / npairs;
  const int pair = work - bh * npairs;
  const int qt_raw = 2 * pair + group;
  const bool valid = qt_raw < qtiles;
  const int qt = valid ? qt_raw : qt_raw - 1;
  const int64_t head = int64_t(bh) * S * kD;

  const char* kg = k + head * 2;
  const char* vg = v + head * 2;
  const int ntiles = S / BN;
  const int kfill = k_fill_offset(lane);
  const int vfill = v_fill_offset(lane);
  // K: row 16kb + col (block 4kb + col/4, row col%4), 16-byte chunk 4*step + g.
  const int k_lane = (col >> 2) * kKBlockPair + ((col & 3) + 4 * g) * 16;
  // V: block 8t + g (+4 for the second read), row col/4 of it, d columns
  // 16db + 4(col%4) .. +3.
  const int v_lane = g * kVBlock + 64 * (col >> 2) + 16 * ((col & 3) >> 1) + 8 * (col & 1);
  // The tensor this wave's group streams from during its softmax phases
  // (K for group B, V for group A).
  const char* const lsrc = group == 1 ? kg : vg;
  const int lfill = group == 1 ? kfill : vfill;

#pragma unroll
  for (int i = 0; i < T::kBlocks / 8; ++i) {
    const int j = 8 * i + wave8;
    __builtin_amdgcn_global_load_lds(kg + j * 1024 + kfill, (lds_void*)(kb0 + j * kKBlockPair), 16, 0, 0);
  }

  // Q fragments: query block qb, 32-dim step: dims 32*step + 8g .. +7.
  const int qrow0 = qt * (64 * QB) + wave * (16 * QB) + col;  // query of block 0; block qb is +16 qb
  bf16x8 qf[QB][4];
  auto load_q = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint4* qp = q + ((head + int64_t(qrow0 + 16 * qb) * kD) >> 3);
#pragma unroll
      for (int step = 0; step < 4; ++step) qf[qb][step] = __builtin_bit_cast(bf16x8, qp[4 * step + g]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // K(1) is issued in every case (through a resource of zero length when
  // there is no K(1): zero fills without a memory access), so that the wait
  // counts below are fixed.
  auto load_k1 = [&]() {
    const __amdgpu_buffer_rsrc_t rs1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kg + kTileBytes), 0, ntiles > 1 ? kTileBytes : 0, kBufferWord3);
#pragma unroll
    for (int i = 0; i < T::kBlocks / 8; ++i) {
      const int j = 8 * i + wave8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs1, (lds_void*)(kb1 + j * kKBlockPair), 16, kfill, j * 1024, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x4 acc[8][QB];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[db][qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float kept[QB];
  f32x4 lacc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // every row takes its first tile's max as its base (alpha = 0 then)
    kept[qb] = -FLT_MAX;
    lacc[qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  asm volatile("" : "+v"(ones));  // keep it in registers, not rebuilt before each use
  // sparse-A index of the row-sum smfmac: rows 0-7 (lanes 0-31 of D) keep
  // the values k%4 in {0, 1} of each group of four, rows 8-15 keep {2, 3}
  int sidx = (lane & 15) < 8 ? 0x4444 : 0xEEEE;
  asm volatile("" : "+v"(sidx));
  f32x4 s[BN / 16][QB];
  bf16x8 pf[QB][BN / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int t = 0; t < BN / 32; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[qb][t][e] = (__bf16)0.0f;

  // The first barrier needs K(0) only (and group A's Q, for its QK(0)
  // right after): group A issues Q before K(1) and waits for all but K(1);
  // group B, whose QK(0) comes one interval later, issues K(1) before its Q
  // and waits for K(0) alone. Each group then runs its own copy of QK(0),
  // so that the waits the compiler adds for Q stay on their own path.
  static_assert(T::kBlocks / 8 == 4 && 4 + 4 * QB <= 15, "the prologue's wait counts");
  if (group == 0) {
    load_q();
    load_k1();
    __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0): K(0) and Q have landed
    barrier();
    qk16_tile<BN, QB>(kb0, k_lane, qf, s);
  } else {
    load_k1();
    load_q();
    // vmcnt(4 + 4 QB) lgkmcnt(0): K(0) has landed
    __builtin_amdgcn_s_waitcnt(0x0070 | (4 + 4 * QB));
    barrier();
    barrier();
    qk16_tile<BN, QB>(kb0, k_lane, qf, s);
  }
  wait_mem();
  barrier();
  float alpha[QB];
  bool rescale;
  pp_v_phase<BN, QB, kEmuEvery, true>(0, group, wave, lsrc, ntiles, lfill, kb0, vb0, c, s, pf, alpha, rescale,
                                kept, lacc, ones, sidx);
  // The wave in its MFMA phase gets the higher issue priority. Without it
  // the SIMD favours the older wave (group A's), so while group A runs its
  // softmax phase it delays group B's MFMAs: an instrumented copy measured
  // group B's MFMA phase ~20% longer than group A's.
  for (int i = 1; i < ntiles; ++i) {
    const bool odd = i & 1;
    char* const k_i = odd ? kb1 : kb0;
    char* const v_other = odd ? vb0 : vb1;
    __builtin_amdgcn_s_setprio(1);
    pp_m_phase<BN, QB>(k_i, v_other, k_lane, v_lane, qf, s, pf, acc, alpha, rescale, false, lacc, ones, sidx);
    __builtin_amdgcn_s_setprio(0);
    pp_v_phase<BN, QB, kEmuEvery, false>(i, group, wave, lsrc, ntiles, lfill, k_i, odd ? vb1 : vb0, c, s, pf, alpha,
                                  rescale, kept, lacc, ones, sidx);
  }
  // The last MFMA phase: PV(ntiles - 1) alone (there is no tile ntiles to
  // score). Kept out of the loop: as a branch inside it, the second copy of
  // the phase made the register allocator spill.
  __builtin_amdgcn_s_setprio(1);
  pp_m_phase<BN, QB, Frags16<BN>::kV>(ntiles & 1 ? kb1 : kb0, ntiles & 1 ? vb0 : vb1, k_lane, v_lane, qf, s, pf, acc,
                                      alpha, rescale, group == 1, lacc, ones, sidx);
  __builtin_amdgcn_s_setprio(0);
  // Group B's last MFMA phase passed no barrier, and group A passes no
  // extra one: the counts match, and each group stores its rows as soon as
  // its own last phase is done (group A while group B runs its last one).
  if (!valid) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // the two row halves of D hold complementary halves of every key sum
    const auto hs = __builtin_amdgcn_permlane32_swap(__float_as_uint(lacc[qb][0]), __float_as_uint(lacc[qb][0]),
                                                     false, false);
    const float ltot = __uint_as_float(hs[0]) + __uint_as_float(hs[1]);
    const float inv = 1.0f / ltot;
    const int qrow = qrow0 + 16 * qb;
    __bf16* orow = o + head + int64_t(qrow) * kD;
    // Lane group g holds dims 16 db + 4g .. +3 of each block db. For the
    // blocks 2p and 2p+1, one 16-lane swap between groups 2h and 2h+1 gives
    // group 2h dims 16(2p) + 8h .. +7 and group 2h+1 dims 16(2p+1) + 8h .. +7:
    // each lane stores 16 bytes, and a row's 64 bytes of the two blocks go
    // out in one instruction.
    const bool odd = g & 1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      bf16x4 ca, cb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ca[i] = (__bf16)(acc[2 * p][qb][i] * inv);
        cb[i] = (__bf16)(acc[2 * p + 1][qb][i] * inv);
      }
      const u32x2 a = __builtin_bit_cast(u32x2, ca), b = __builtin_bit_cast(u32x2, cb);
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // [0]: a with groups 1 and 3 replaced by b of groups 0 and 2;
        // [1]: b with groups 0 and 2 replaced by a of groups 1 and 3
        const auto sw = __builtin_amdgcn_permlane16_swap(a[i], b[i], false, false);
        w[i] = odd ? sw[0] : a[i];
        w[2 + i] = odd ? b[i] : sw[1];
      }
      *reinterpret_cast<u32x4*>(orow + 32 * p + 16 * (g & 1) + 8 * (g >> 1)) = w;
    }
    if (g == 0) lse[int64_t(bh) * S + qrow] = (kept[qb] + __log2f(ltot)) * kLn2;
  }
}

}  // namespace

#ifndef ATTN_PP_BN
#define ATTN_PP_BN 128
#endif
#ifndef ATTN_PP_MIN_WGS
#define ATTN_PP_MIN_WGS 256
#endif
// PAIR256_EXP2EMU: one exponential in this many on the FMA pipe.
#ifndef ATTN_EXP2_EMU_EVERY
#define ATTN_EXP2_EMU_EVERY 4
#endif


namespace {
// PAIR256: two 128-row query tiles per workgroup (two 16-query blocks per
// wave); PAIR128: two 64-row tiles (one block per wave), for grids too
// small to fill the GPU with 256-row workgroups. TILE128: one 128-row tile.
bool is_pair(int variant) {
  return variant == ATTN_VARIANT_PAIR256 || variant == ATTN_VARIANT_PAIR256_EXP2EMU ||
         variant == ATTN_VARIANT_PAIR128;
}
int pair_rows(int variant) { return variant == ATTN_VARIANT_PAIR128 ? 64 : 128; }
int64_t workgroups(int B, int H, int S, int variant) {
  if (!is_pair(variant)) return int64_t(B) * H * (S / kBM);
  const int tiles = S / pair_rows(variant);
  return int64_t(B) * H * ((tiles + 1) / 2);
}
}  // namespace

int64_t launch_threads(int B, int H, int S, int variant) {
  return workgroups(B, H, S, variant) * (is_pair(variant) ? 2 * kThreads : kThreads);
}

// PAIR256 once its workgroups (pairs of 128-row tiles) fill the GPU's CUs
// once; below that PAIR128 (pairs of 64-row tiles), down to launches of a
// handful of workgroups, which one 128-row tile per workgroup serves a little
// faster. Measured: from 256 PAIR256 workgroups up PAIR256 is fastest; below,
// PAIR128 beats TILE128 by 13-48% at 32-256 workgroups; at 2 workgroups
// (S = 256, one head) TILE128 is 5% ahead. A grid so large that PAIR256's
// launch would reach 2^32 threads (only possible when S / 128 is odd, which
// leaves half of the last workgroup of each head idle) takes TILE128, which
// needs fewer threads.
int pick_variant(int B, int H, int S) {
  const int64_t pair_wgs = int64_t(B) * H * ((S / kBM + 1) / 2);
  const int64_t half_pair_wgs = int64_t(B) * H * (S / (2 * 64));
  if (pair_wgs >= ATTN_PP_MIN_WGS)
    return launch_threads(B, H, S, ATTN_VARIANT_PAIR256) < (int64_t(1) << 32) ? ATTN_VARIANT_PAIR256
                                                                             : ATTN_VARIANT_TILE128;
  if (half_pair_wgs >= 16) return ATTN_VARIANT_PAIR128;
  return ATTN_VARIANT_TILE128;
}

namespace {
template <class T>
struct same_type {
  using type = T;
};
// hipLaunchKernel with the kernel's own parameter types: returns the status
// of this launch (not an error left behind by earlier runtime calls, as
// hipGetLastError after the <<<>>> form would).
template <typename... KArgs>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         typename same_type<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}
}  // namespace

hipError_t launch(const Params& p, hipStream_t stream) {
  constexpr int BN = ATTN_BN;
  const int qtiles = p.S / kBM;
  const float c = p.scale * kLog2e;
  const auto* q = static_cast<const uint4*>(p.q);
  const auto* k = static_cast<const char*>(p.k);
  const auto* v = static_cast<const char*>(p.v);
  auto* o = static_cast<__bf16*>(p.o);
  const int nwg = int(workgroups(p.B, p.H, p.S, p.variant));  // below 2^32 / 256 (checked)
  if (is_pair(p.variant)) {
    const int tiles = p.S / pair_rows(p.variant);
    const int npairs = (tiles + 1) / 2;
    auto kernel = p.variant == ATTN_VARIANT_PAIR256   ? attn_fwd_pingpong_kernel<ATTN_PP_BN, 2, 0>
                  : p.variant == ATTN_VARIANT_PAIR128 ? attn_fwd_pingpong_kernel<ATTN_PP_BN, 1, 0>
                                                      : attn_fwd_pingpong_kernel<ATTN_PP_BN, 2, ATTN_EXP2_EMU_EVERY>;
    return launch_kernel(kernel, dim3(nwg), dim3(2 * kThreads), stream, q, k, v, o, p.lse, p.S, tiles,
                         npairs, nwg, c);
  }
  return launch_kernel(attn_fwd_kernel<BN>, dim3(nwg), dim3(kThreads), stream, q, k, v, o, p.lse, p.S,
                       qtiles, nwg, c);
}

}  // namespace attn_detail
