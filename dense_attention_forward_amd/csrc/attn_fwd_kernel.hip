// Dense, non-causal, bf16, head_dim-128 attention forward for gfx950 (MI355X).
//
// Method: "B200 attention kernel from scratch to ~SOTA in 60 figures",
// Chapter 1 (one workgroup per 128-row output tile, a sequential K/V loop
// inside it, online softmax of section B), Chapter 8 (base-2 exponent with
// scale*log2(e) folded into the score scale; the max is taken over raw
// scores and scaled once), Chapter 11 (the O accumulator is rescaled only
// when a row's max grows by >= 8 in base-2 units, decided per wave).
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
//    16-column block of the row-major V tile across each 16-lane group.
//  * K and V tiles are staged in LDS with 16-byte XOR swizzles chosen so
//    that the MFMA operand reads are bank-conflict free; the next tile is
//    prefetched into registers while the current one is consumed.
//  * Workgroups are renumbered so that each XCD (blocks are dispatched to
//    the 8 XCDs round-robin) processes a contiguous range of (b, h, tile)
//    work items, keeping one head's K/V in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "attn_fwd_launch.h"

namespace attn_detail {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;         // head dimension
constexpr int kBM = 128;        // query rows per workgroup
constexpr int kChunks = kD / 8; // 16-byte chunks per K/V row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRebaseLog2 = 8.0f;  // rebase threshold in base-2 exponent units

// K tile: chunk c of key row r is stored at slot c ^ (r % 16). The QK^T A
// operand read has 16 consecutive rows at one chunk per 16 lanes, which
// this spreads over all 64 banks.
__device__ __forceinline__ int k_slot(int r, int c) { return r * kChunks + (c ^ (r & 15)); }
// V tile: chunk c of key row r is stored at slot c ^ 4*(r % 4). A transposed
// read touches 4 consecutive rows x 2 chunks per 16 lanes (and 4 rows x 4
// chunks per 32 lanes), which this places in distinct banks.
__device__ __forceinline__ int v_slot(int r, int c) { return r * kChunks + (c ^ ((r & 3) << 2)); }

typedef __attribute__((address_space(3))) void lds_void;

// Issues the direct-to-LDS loads of one BN-row K (or V) tile: each
// global_load_lds_dwordx4 writes 64 lanes x 16 bytes to consecutive LDS
// slots, so lane l of wave w, load i fills slot (4i + w) * 64 + l; the lane
// fetches the global chunk that the swizzle maps to that slot.
template <int BN, bool kIsK>
__device__ __forceinline__ void load_tile(const char* __restrict__ g, uint4* lds, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < BN / 16; ++i) {
    const int blk = 4 * i + wave;            // 64-slot block = 4 rows
    const int r = 4 * blk + (lane >> 4);     // key row in the tile
    const int p = lane & 15;                 // physical chunk slot in the row
    const int ch = kIsK ? (p ^ (r & 15)) : (p ^ ((r & 3) << 2));  // logical chunk
    __builtin_amdgcn_global_load_lds(g + r * 256 + ch * 16, (lds_void*)(lds + blk * 64), 16, 0, 0);
  }
}

struct Softmax {
  float kept;  // kept row max, base-2 units of scaled scores
  float lsum;  // this half-wave's share of the row sum
};

// One K/V tile: S^T = K Q^T, online-softmax update, O^T += V^T P^T.
template <int BN>
__device__ __forceinline__ void tile_step(const uint4* ksm, const char* vsm, const bf16x8 (&qf)[8],
                                          f32x16 (&acc)[4], Softmax& st_, float c, int n, int h,
                                          int tr_row, int tr_col) {
  constexpr int kBlocks = BN / 32;  // 32-key score blocks per tile
  constexpr int kSteps = BN / 16;   // 16-key PV steps per tile

  // S^T block cb: keys 32cb + 8j + 4h + i, query n.
  f32x16 st[kBlocks];
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) st[cb][i] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, ksm[k_slot(32 * cb + n, 2 * kk + h)]);
      st[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], st[cb], 0, 0, 0);
    }
  }

  // Row max of raw scores, scaled once into base-2 units.
  float mx = -FLT_MAX;
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[cb][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float cand = fmaxf(st_.kept, mx * c);
  const bool need = (cand - st_.kept) >= kRebaseLog2;
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(st_.kept - cand) : 1.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;
    st_.lsum *= alpha;
    st_.kept = need ? cand : st_.kept;
  }

  // P = 2^(s*c - kept); the row sum takes the unrounded values, P.V the
  // bf16 ones. Step t's operand: slots 0..3 <- block t/2, j = 2(t%2);
  // slots 4..7 <- j = 2(t%2)+1.
  bf16x8 pf[kSteps];
  float ps = 0.0f;
  const float kept = st_.kept;
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[cb][4 * j + i], c, -kept));
        ps += p;
        pf[2 * cb + (j >> 1)][(j & 1) * 4 + i] = (__bf16)p;
      }
  st_.lsum += ps;

  // O^T[d-block b] += V^T[b, step t] . P^T[step t]
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int col = 32 * b + tr_col;
      const int r0 = 16 * t + tr_row, r1 = r0 + 8;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vsm + v_slot(r0, col >> 3) * 16 + (col & 7) * 2));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vsm + v_slot(r1, col >> 3) * 16 + (col & 7) * 2));
      const i16x8 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16), pf[t],
                                                       acc[b], 0, 0, 0);
    }
  }
}

template <int BN>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const uint4* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int S, int qtiles, int nwg, float c) {
  static_assert(BN % 32 == 0 && BN % 16 == 0, "tile shape");
  constexpr int kTileBytes = BN * kD * 2;
  // Two K/V buffers as separate objects, so LDS reads of one buffer need
  // not wait for the direct-to-LDS loads filling the other.
  __shared__ uint4 k0[BN * kChunks], v0[BN * kChunks];
  __shared__ uint4 k1[BN * kChunks], v1[BN * kChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  load_tile<BN, true>(kg, k0, wave, lane);
  load_tile<BN, false>(vg, v0, wave, lane);

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
  Softmax sm{-FLT_MAX, 0.0f};

  // Per-lane parts of the transposed V read address (see v_slot).
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int jt = 0; jt < ntiles; jt += 2) {
    __syncthreads();  // tile jt is in buffer 0; everyone is done with buffer 1
    if (jt + 1 < ntiles) {
      load_tile<BN, true>(kg + int64_t(jt + 1) * kTileBytes, k1, wave, lane);
      load_tile<BN, false>(vg + int64_t(jt + 1) * kTileBytes, v1, wave, lane);
    }
    tile_step<BN>(k0, reinterpret_cast<const char*>(v0), qf, acc, sm, c, n, h, tr_row, tr_col);
    if (jt + 1 >= ntiles) break;
    __syncthreads();  // tile jt+1 is in buffer 1; everyone is done with buffer 0
    if (jt + 2 < ntiles) {
      load_tile<BN, true>(kg + int64_t(jt + 2) * kTileBytes, k0, wave, lane);
      load_tile<BN, false>(vg + int64_t(jt + 2) * kTileBytes, v0, wave, lane);
    }
    tile_step<BN>(k1, reinterpret_cast<const char*>(v1), qf, acc, sm, c, n, h, tr_row, tr_col);
  }

  // Epilogue: O = O^T / l -> bf16; lane holds dims 32b + 8j + 4h + 0..3.
  const float ltot = sm.lsum + __shfl_xor(sm.lsum, 32);
  const float inv = 1.0f / ltot;
  __bf16* orow = o + head + int64_t(qrow) * kD;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc[b][4 * j + i] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * j + 4 * h) = w;
    }
  if (h == 0) lse[int64_t(bh) * S + qrow] = (sm.kept + __log2f(ltot)) * kLn2;
}

}  // namespace

hipError_t launch(const Params& p, hipStream_t stream) {
  constexpr int BN = 64;
  const int qtiles = p.S / kBM;
  const int nwg = p.B * p.H * qtiles;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL(attn_fwd_kernel<BN>, dim3(nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(p.q), static_cast<const char*>(p.k),
                     static_cast<const char*>(p.v), static_cast<__bf16*>(p.o), p.lse, p.S,
                     qtiles, nwg, c);
  return hipGetLastError();
}

}  // namespace attn_detail
