// Dense, non-causal, bf16, head_dim-128 attention forward for gfx950 (MI355X).
//
// Method: "B200 attention kernel from scratch to ~SOTA in 60 figures",
// Chapter 1 (one workgroup per 128-row output tile, a sequential K/V loop
// inside it, online softmax of section B), Chapter 8 (base-2 exponent with
// scale*log2(e) folded into the score scale; the max is taken over raw
// scores and scaled once), Chapter 11 (the O accumulator is rescaled only
// when a row's max grows by >= 8 in base-2 units, decided per wave),
// Chapters 6-7 (K and V move through separate double buffers, and the
// next tile's QK^T is issued while the current tile's softmax runs).
//
// gfx950 mapping (not the article's B200 mapping):
//  * Workgroup = 4 wave64s; wave w owns query rows 32w..32w+31 of the tile.
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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;         // head dimension
constexpr int kBM = 128;        // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRebaseLog2 = 8.0f;  // rebase threshold in base-2 exponent units

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
// K: the slot of (row 4j + rr, 16-byte chunk 2kk + h) is rr + 4h + 8kk, and
// blocks are 1088 bytes apart (64 bytes of padding). The QK^T A-operand
// read of step kk has lane (n, h) at block n/4, slot (n%4) + 4h + 8kk: 16
// lanes of one half-wave cover 4 blocks x 4 rows, whose bank groups
// 4*(block%4) + rr + 4h + 8kk (mod 16) are all distinct.
constexpr int kKBlock = 1088;
// V: the slot of (row 4j + q, chunk 4b + x) is 16b + 4q + x, blocks 1 KB
// apart. The transposed read of d-block b touches, per half-wave, the 4
// rows of one block at chunks 4b..4b+3: 16 consecutive slots, all banks
// once.
constexpr int kVBlock = 1024;

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

// Raw row max of a score tile, over both half-waves.
template <int BN>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[BN / 32]) {
  float mx = -FLT_MAX;
#pragma unroll
  for (int cb = 0; cb < BN / 32; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[cb][i]);
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// P = 2^(s*c - kept) as the PV B operand; returns the sum of the unrounded
// values. Step t's operand: slots 0..3 <- block t/2, j = 2(t%2); slots
// 4..7 <- j = 2(t%2)+1.
template <int BN>
__device__ __forceinline__ float exp_tile(const f32x16 (&s)[BN / 32], float c, float kept,
                                          bf16x8 (&pf)[BN / 16]) {
  float ps = 0.0f;
#pragma unroll
  for (int cb = 0; cb < BN / 32; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][4 * j + i], c, -kept));
        ps += p;
        pf[2 * cb + (j >> 1)][(j & 1) * 4 + i] = (__bf16)p;
      }
  return ps;
}

// O^T[d-block b] += V^T[b, step t] . P^T[step t] for one V tile.
template <int BN>
__device__ __forceinline__ void pv_tile(const char* vsm, int v_lane, const bf16x8 (&pf)[BN / 16],
                                        f32x16 (&acc)[4]) {
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
  }
}

// Online-softmax base update for a new tile max (raw units): rebase when
// the scaled max exceeds the kept base by >= 8, rescaling O and the row sum
// only if some lane of the wave rebased.
__device__ __forceinline__ void update_base(float raw_max, float c, float& kept, float& lsum,
                                            f32x16 (&acc)[4]) {
  const float cand = fmaxf(kept, raw_max * c);
  const bool need = (cand - kept) >= kRebaseLog2;
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(kept - cand) : 1.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;
    lsum *= alpha;
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
                                             f32x16 (&acc)[4], float& kept, float& lsum) {
  constexpr int kTileBytes = BN * kD * 2;
  if (jt + 2 < ntiles) load_tile<BN, kKBlock>(kg + int64_t(jt + 2) * kTileBytes, kfill, k_cur, wave);
  if (jt + 1 < ntiles) load_tile<BN, kVBlock>(vg + int64_t(jt + 1) * kTileBytes, vfill, v_next, wave);

  bf16x8 pf[BN / 16];
  lsum += exp_tile<BN>(s, c, kept, pf);
  // QK^T of the next tile, issued without a branch so it can interleave
  // with the exponentials above; on the last tile it reads a stale (but
  // in-bounds) buffer and its result is dropped.
  qk_tile<BN>(k_next, k_lane, qf, sn);
  pv_tile<BN>(v_cur, v_lane, pf, acc);
  if (jt + 1 < ntiles) update_base(tile_max<BN>(sn), c, kept, lsum, acc);
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
  float lsum = 0.0f;      // this half-wave's share of the row sum

  f32x16 s0[BN / 32], s1[BN / 32];
  __syncthreads();  // K0, V0 (and K1) are in LDS
  qk_tile<BN>(kb0, k_lane, qf, s0);
  update_base(tile_max<BN>(s0), c, kept, lsum, acc);
  __syncthreads();  // everyone is done reading K0

  // Iterations alternate the roles of the two K buffers, the two V buffers
  // and the two score register sets.
  for (int jt = 0; jt < ntiles; jt += 2) {
    kv_iteration<BN>(jt, ntiles, kg, vg, kfill, vfill, wave, kb0, kb1, vb0, vb1, k_lane, v_lane, qf,
                     c, s0, s1, acc, kept, lsum);
    if (jt + 1 >= ntiles) break;
    kv_iteration<BN>(jt + 1, ntiles, kg, vg, kfill, vfill, wave, kb1, kb0, vb1, vb0, k_lane, v_lane,
                     qf, c, s1, s0, acc, kept, lsum);
  }

  // Epilogue: O = O^T / l -> bf16; lane holds dims 32b + 8j + 4h + 0..3.
  const float ltot = lsum + __shfl_xor(lsum, 32);
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
// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for loads that are meant to stay in flight across it).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// K fragment for QK step u (u interleaves the 32-key blocks so consecutive
// MFMAs feed independent accumulators): block u % (BN/32), dims chunk u / (BN/32).
template <int BN>
__device__ __forceinline__ bf16x8 k_frag(const char* ksm, int k_lane, int u) {
  constexpr int kCB = BN / 32;
  return *reinterpret_cast<const bf16x8*>(ksm + k_lane + (u % kCB) * 8 * kKBlock + (u / kCB) * 128);
}
// V^T fragment for PV step u: key step u / 4, d-block u % 4.
__device__ __forceinline__ bf16x8 v_frag(const char* vsm, int v_lane, int u) {
  const char* p0 = vsm + v_lane + (u >> 2) * 4 * kVBlock + (u & 3) * 256;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + 2 * kVBlock));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The MFMA work of one phase: QK of a K tile into s and/or PV of a V tile
// into acc, one MFMA of each per step, with the operands of step u+1
// fetched from LDS while step u issues (scheduling barriers keep the
// compiler from hoisting every fetch and running out of registers).
template <int BN, bool kQK, bool kPV>
__device__ __forceinline__ void mma_steps(const char* ksm, const char* vsm, int k_lane, int v_lane,
                                          const bf16x8 (&qf)[8], f32x16 (&s)[BN / 32],
                                          const bf16x8 (&pf)[BN / 16], f32x16 (&acc)[4]) {
  constexpr int kSteps = BN / 4;  // = 8 * BN/32 QK MFMAs = 4 * BN/16 PV MFMAs
  constexpr int kCB = BN / 32;
  if (kQK) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[cb][i] = 0.0f;
  }
  bf16x8 ka = {}, va = {};
  if (kQK) ka = k_frag<BN>(ksm, k_lane, 0);
  if (kPV) va = v_frag(vsm, v_lane, 0);
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    bf16x8 kn = {}, vn = {};
    if (u + 1 < kSteps) {
      if (kQK) kn = k_frag<BN>(ksm, k_lane, u + 1);
      if (kPV) vn = v_frag(vsm, v_lane, u + 1);
    }
    if (kQK) s[u % kCB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[u / kCB], s[u % kCB], 0, 0, 0);
    if (kPV) acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[u >> 2], acc[u & 3], 0, 0, 0);
    ka = kn;
    va = vn;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// MFMA phase i >= 1 of the eight-wave kernel: PV(i-1) and QK(i), then
// publish this wave's finished loads and pass a barrier. In the last phase
// (i == ntiles) the QK reads a stale but in-bounds buffer and its result is
// never used; issuing it keeps the phase branch-free.
template <int BN>
__device__ __forceinline__ void pp_m_phase(const char* kcur, const char* vprev, int k_lane,
                                           int v_lane, const bf16x8 (&qf)[8], f32x16 (&s)[BN / 32],
                                           const bf16x8 (&pf)[BN / 16], f32x16 (&acc)[4]) {
  mma_steps<BN, true, true>(kcur, vprev, k_lane, v_lane, qf, s, pf, acc);
  wait_mem();
  barrier();
}

// Softmax phase i: group B first issues the loads of K(i+2) (into the
// buffer K(i) left) and V(i+1); then the base update, which rescales O
// (already holding PV(i-1)) if needed, and P(i).
template <int BN>
__device__ __forceinline__ void pp_v_phase(int i, int ntiles, int group, int wave, const char* kg,
                                           const char* vg, int kfill, int vfill, char* kfree,
                                           char* vnext, float c, const f32x16 (&s)[BN / 32],
                                           bf16x8 (&pf)[BN / 16], f32x16 (&acc)[4], float& kept,
                                           float& lsum) {
  constexpr int kTileBytes = BN * kD * 2;
  if (group == 1) {
    if (i + 2 < ntiles) load_tile<BN, kKBlock>(kg + int64_t(i + 2) * kTileBytes, kfill, kfree, wave);
    if (i + 1 < ntiles) load_tile<BN, kVBlock>(vg + int64_t(i + 1) * kTileBytes, vfill, vnext, wave);
  }
  update_base(tile_max<BN>(s), c, kept, lsum, acc);
  lsum += exp_tile<BN>(s, c, kept, pf);
  barrier();
}

// Eight-wave variant: two 4-wave groups own two consecutive 128-row Q tiles
// of one head and share every K/V tile (the article's two-Q-tile CTA,
// Chapter 5). Barriers make the groups alternate: while one group runs
// its MFMA phase [PV(i-1), QK(i)] the other runs its softmax phase on the
// SIMD it shares (the role split of Chapters 4 and 12, done here by
// phase-shifting two groups of identical waves instead of specialised warps).
//
// Group A runs M(0) V(0) M(1) V(1) ... M(n); group B starts one barrier
// later, so interval 2i+1 holds A's V(i) and B's M(i), interval 2i+2 A's
// M(i+1) and B's V(i). K(i) and V(i) live in buffer i%2; K(i+2) and V(i+1)
// are loaded by group B at the start of its V(i) (their buffers' last
// readers finished by then) and waited for at the end of its M(i+1), one
// barrier before group A first reads them.
template <int BN>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pingpong_kernel(const uint4* __restrict__ q, const char* __restrict__ k,
                              const char* __restrict__ v, __bf16* __restrict__ o,
                              float* __restrict__ lse, int S, int qtiles, int npairs, int nwg,
                              float c) {
  static_assert(BN % 64 == 0, "tile shape");
  constexpr int kTileBytes = BN * kD * 2;
  using T = Tiles<BN>;
  __shared__ uint4 k0[T::kKBytes / 16], k1[T::kKBytes / 16];
  __shared__ uint4 v0[T::kVBytes / 16], v1[T::kVBytes / 16];
  char* const kb0 = reinterpret_cast<char*>(k0);
  char* const kb1 = reinterpret_cast<char*>(k1);
  char* const vb0 = reinterpret_cast<char*>(v0);
  char* const vb1 = reinterpret_cast<char*>(v1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave8 >> 2;  // 0 = A, 1 = B
  const int wave = wave8 & 3;    // wave within the group
  const int n = lane & 31;
  const int h = lane >> 5;

  const int bid = blockIdx.x;
  const int per = nwg >> 3;
  const int work = bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bh = work / npairs;
  const int pair = work - bh * npairs;
  const int qt_raw = 2 * pair + group;
  const bool valid = qt_raw < qtiles;       // an odd tile count leaves B's last tile empty
  const int qt = valid ? qt_raw : qt_raw - 1;  // then B recomputes A's tile and stores nothing
  const int64_t head = int64_t(bh) * S * kD;

  const char* kg = k + head * 2;
  const char* vg = v + head * 2;
  const int ntiles = S / BN;
  const int kfill = k_fill_offset(lane);
  const int vfill = v_fill_offset(lane);
  const int k_lane = (n >> 2) * kKBlock + ((n & 3) + 4 * h) * 16;
  const int v_lane = h * kVBlock + 64 * ((lane & 15) >> 2) +
                     16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);

  // Prologue loads by all eight waves: K(0), V(0), K(1).
  {
    // Wave w8 of 8 issues blocks w8, w8+8, ...; reuse the 4-wave loader on
    // half-tiles.
#pragma unroll
    for (int i = 0; i < T::kBlocks / 8; ++i) {
      const int j = 8 * i + wave8;
      __builtin_amdgcn_global_load_lds(kg + j * 1024 + kfill, (lds_void*)(kb0 + j * kKBlock), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vg + j * 1024 + vfill, (lds_void*)(vb0 + j * kVBlock), 16, 0, 0);
      if (ntiles > 1)
        __builtin_amdgcn_global_load_lds(kg + kTileBytes + j * 1024 + kfill,
                                         (lds_void*)(kb1 + j * kKBlock), 16, 0, 0);
    }
  }

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
  float kept = -FLT_MAX;
  float lsum = 0.0f;
  f32x16 s[BN / 32];
  bf16x8 pf[BN / 16];
#pragma unroll
  for (int t = 0; t < BN / 16; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) pf[t][i] = (__bf16)0.0f;

  __syncthreads();  // prologue tiles are in LDS
  if (group == 1) barrier();  // phase shift: B starts one interval later

  // M(0) is QK(0) alone; after it every MFMA phase i holds PV(i-1) and
  // QK(i). Buffers alternate with i; the loop is unrolled by two so that
  // each half names its buffers statically.
  mma_steps<BN, true, false>(kb0, vb0, k_lane, v_lane, qf, s, pf, acc);
  wait_mem();
  barrier();
  pp_v_phase<BN>(0, ntiles, group, wave, kg, vg, kfill, vfill, kb0, vb1, c, s, pf, acc, kept, lsum);
  for (int i = 1;; i += 2) {
    pp_m_phase<BN>(kb1, vb0, k_lane, v_lane, qf, s, pf, acc);
    if (i == ntiles) break;
    pp_v_phase<BN>(i, ntiles, group, wave, kg, vg, kfill, vfill, kb1, vb0, c, s, pf, acc, kept, lsum);
    pp_m_phase<BN>(kb0, vb1, k_lane, v_lane, qf, s, pf, acc);
    if (i + 1 == ntiles) break;
    pp_v_phase<BN>(i + 1, ntiles, group, wave, kg, vg, kfill, vfill, kb0, vb1, c, s, pf, acc, kept,
                   lsum);
  }
  if (group == 0) barrier();  // matches B's phase-shift barrier

  if (!valid) return;
  const float ltot = lsum + __shfl_xor(lsum, 32);
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

}  // namespace

#ifndef ATTN_PP_BN
#define ATTN_PP_BN 64
#endif
#ifndef ATTN_PP_MIN_WGS
#define ATTN_PP_MIN_WGS 512
#endif


int pick_variant(int B, int H, int S) {
  const int64_t pair_wgs = int64_t(B) * H * ((S / kBM + 1) / 2);
  return pair_wgs >= ATTN_PP_MIN_WGS ? ATTN_VARIANT_PAIR256 : ATTN_VARIANT_TILE128;
}

hipError_t launch(const Params& p, hipStream_t stream) {
  constexpr int BN = ATTN_BN;
  const int qtiles = p.S / kBM;
  const float c = p.scale * kLog2e;
  if (p.variant == ATTN_VARIANT_PAIR256) {
    const int npairs = (qtiles + 1) / 2;
    const int nwg = int(int64_t(p.B) * p.H * npairs);
    hipLaunchKernelGGL(attn_fwd_pingpong_kernel<ATTN_PP_BN>, dim3(nwg), dim3(2 * kThreads), 0, stream,
                       static_cast<const uint4*>(p.q), static_cast<const char*>(p.k),
                       static_cast<const char*>(p.v), static_cast<__bf16*>(p.o), p.lse, p.S,
                       qtiles, npairs, nwg, c);
    return hipGetLastError();
  }
  const int nwg = p.B * p.H * qtiles;
  hipLaunchKernelGGL(attn_fwd_kernel<BN>, dim3(nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(p.q), static_cast<const char*>(p.k),
                     static_cast<const char*>(p.v), static_cast<__bf16*>(p.o), p.lse, p.S,
                     qtiles, nwg, c);
  return hipGetLastError();
}

}  // namespace attn_detail
