// Eight-wave pipelined bf16 MFMA main loop for the expert GEMMs.
//
// Tile: BW = 256 weight rows x BT = 320 token rows, eight waves (512
// threads, two per SIMD). Ten 32-row token sub-tiles cover an expert of up to
// 320 rows in one block, so at the DeepSeek-V3 shape (256 rows per expert on
// average) every expert's weights stream from HBM once; with two waves per
// SIMD one wave's MFMAs run while the other waits on LDS or a barrier.
//
// Wave w: weight quarter ww = w & 3 (two 32-row weight sub-tiles whose tile
// rows the caller chooses: the gate and the matching up rows for the gate/up
// projection, 64 consecutive rows for the down projection) and token half
// wt = w >> 2 (token sub-tiles wt, wt + 2, ..., up to five): 2 x 5 sub-tiles
// of 32x32x16 MFMAs, 160 accumulator registers. Only the MS live token
// sub-tiles (compile time) are computed.
//
// Both operands stream from global memory straight into LDS with
// buffer_load_dwordx4 ... lds through a ring of four stages of 32 K-elements
// (36 KB each): weight rows from the tiled layout of moe_tile_weights_bf16 (a
// stage's 16 KB is one contiguous block, the LDS image itself) or row-major,
// token rows by their source-row offsets (the gather fused in). LDS rows are
// 64 bytes, 16-byte chunks XOR-swizzled by (row >> 2) & 3 as in gemm_pipe.h.
//
// Schedule of stage kt per wave: read the step-1 fragments; the step-0 MFMAs
// with the token loads of stage kt + 2 spread among them; wait until stage
// kt + 1 has landed + barrier; read stage kt + 1's step-0 fragments; the
// step-1 MFMAs with the weight loads of stage kt + 3 spread among them.
// Weight loads of stage s go into the buffer of stage s - 4, token loads of
// stage s into that of s - 4 as well, and both follow a barrier after which
// no wave reads that buffer again (the argument of gemm_pipe.h, unchanged by
// the wave count).
#pragma once

#include "common.h"
#include "gemm_pipe.h"

namespace moe {

template <bool TILED_>
struct W8 {
  static constexpr int BW = 256, BT = 320, BK = 32, NS = 4, NT = 512, NWAVE = 8;
  static constexpr bool TILED = TILED_;
  static constexpr int TW = 2, TT = 5;                       // 32x32 sub-tiles per wave
  static constexpr int MAXSUB = BT / 32;                     // token sub-tiles per tile
  static constexpr int ROWB = BK * 2;                        // bytes per row per stage
  static constexpr int W_BYTES = BW * ROWB, T_BYTES = BT * ROWB, STAGE = W_BYTES + T_BYTES;
  static constexpr int WL = W_BYTES / 16 / NT;               // weight loads per thread per stage (2)
  static constexpr int TU = T_BYTES / 1024;                  // 1 KB token load units per stage (20)
  static constexpr int TLMAX = (TU + NWAVE - 1) / NWAVE;     // token load slots per thread (3)
  static constexpr int LDS_BYTES = NS * STAGE;
  static_assert(WL * NT * 16 == W_BYTES, "weight stage must split evenly over the threads");
};

// Token load slots of a stage and their count on every wave: slot q of wave w
// loads unit q * 8 + w (tile rows 16 u .. 16 u + 15) when that unit exists.
__device__ __forceinline__ int w8_unit(int q) { return q * 8 + (threadIdx.x >> 6); }
template <int LT>
constexpr int w8_min_token_loads() {
  return LT * 8 <= W8<false>::TU ? LT : LT - 1;      // the waves with the fewest units in their last slot
}

// threadIdx.x behind an opaque copy: lane-derived per-tile values computed from it are recomputed for
// every tile instead of being hoisted out of a persistent kernel's tile loop (where each would hold a
// register for the whole kernel).
__device__ __forceinline__ int w8_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Token load unit of slot q, tile row and logical 16-byte K chunk of this thread's load in unit u
// (tid: the thread index, from w8_tid in per-tile set-up code).
__device__ __forceinline__ int w8_unit(int q, int tid) { return q * 8 + (tid >> 6); }
__device__ __forceinline__ int w8_load_row(int u, int tid) { return u * 16 + ((tid & 63) >> 2); }
__device__ __forceinline__ int w8_load_chunk(int u, int tid) { return (tid & 3) ^ ((w8_load_row(u, tid) >> 2) & 3); }

struct W8Rows {
  __amdgpu_buffer_rsrc_t wrs, trs;
  uint32_t ow[2];       // weight loads (row-major weights only: row * K * 2 + chunk * 16)
  uint32_t ot[3];       // token loads: source row * K * 2 + chunk * 16
};

// Weight loads are non-temporal: a tile's weights are read once, and marking them for early eviction
// keeps the token rows, which the block's other output tiles read again, in L2. kCachePolicyNT is the
// cache-policy operand of a gfx950 buffer load with its nt bit (bit 1) set.
constexpr int kCachePolicyNT = 2;
template <class P>
__device__ __forceinline__ void w8_issue_w(const W8Rows& r, uint8_t* st, int kb, int q) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t vo = P::TILED ? static_cast<uint32_t>(((q * 8 + w) * 64 + (threadIdx.x & 63)) * 16) : r.ow[q];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.wrs, (lds_void_t*)(st + (q * 8 + w) * 1024), 16, vo,
                                           P::TILED ? kb * (P::W_BYTES / P::ROWB) : kb, 0, kCachePolicyNT);
#endif
}

template <class P>
__device__ __forceinline__ void w8_issue_t(const W8Rows& r, uint8_t* st, int kb, int q) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int u = __builtin_amdgcn_readfirstlane(w8_unit(q));
  if (u < P::TU)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.trs, (lds_void_t*)(st + P::W_BYTES + u * 1024), 16, r.ot[q], kb, 0, 0);
#endif
}

template <int MS>
struct W8Frags {
  bf16x8 w[2];
  bf16x8 t[MS > 0 ? MS : 1];
};

// Per-lane LDS byte offsets of the wave's fragments within a stage (step 0;
// step 1 flips bit 5): weight sub-tiles at tile rows wr0, wr1; token sub-tile
// i at tile rows 32 (2 i + wt).
struct W8Offs {
  int w0, w1, t;
};

__device__ __forceinline__ W8Offs w8_offsets(int wr0, int wr1) {
  const int tid = w8_tid();
  const int l = tid & 63, wt = tid >> 8;
  const int cofs = ((l >> 5) ^ (((l & 31) >> 2) & 3)) * 16;
  return {(wr0 + (l & 31)) * 64 + cofs, (wr1 + (l & 31)) * 64 + cofs,
          W8<false>::W_BYTES + (wt * 32 + (l & 31)) * 64 + cofs};
}

template <int MS>
__device__ __forceinline__ void w8_read(W8Frags<MS>& f, const uint8_t* st, const W8Offs& o, int flip) {
  f.w[0] = *reinterpret_cast<const bf16x8*>(st + (o.w0 ^ flip));
  f.w[1] = *reinterpret_cast<const bf16x8*>(st + (o.w1 ^ flip));
#pragma unroll
  for (int i = 0; i < MS; ++i) f.t[i] = *reinterpret_cast<const bf16x8*>(st + ((o.t + i * 64 * 64) ^ flip));
}

// The 2 * MS MFMAs of one K16 step with L loads spread among them (load q
// before MFMA q * M / L). PART 1: weight loads of stage kb; PART 2: token loads.
template <class P, int MS, int LT, int PART>
__device__ __forceinline__ void w8_mma_loads(const W8Frags<MS>& f, f32x16 (&acc)[2][5], const W8Rows& r,
                                             uint8_t* st, int kb) {
  constexpr int M = 2 * MS;
  constexpr int L = PART == 0 ? 0 : (PART == 1 ? P::WL : LT);
#pragma unroll
  for (int m = 0; m < (M > L ? M : L); ++m) {
#pragma unroll
    for (int q = 0; q < L; ++q)
      if ((M == 0 && q == m) || (M > 0 && q * M / (L > 0 ? L : 1) == m)) {
        if (PART == 1) w8_issue_w<P>(r, st, kb, q);
        else w8_issue_t<P>(r, st, kb, q);
        sched_fence();
      }
    if (m < M) acc[m & 1][m >> 1] = mfma_32x32x16_bf16(f.w[m & 1], f.t[m >> 1], acc[m & 1][m >> 1]);
  }
  sched_fence();
}

template <class P, int MS, int LT, bool ISSUE_B, int WAIT, bool ISSUE_A>
__device__ __forceinline__ void w8_iteration(const W8Rows& rows, uint8_t* lds, int kt, const W8Offs& o,
                                             W8Frags<MS>& f0, W8Frags<MS>& f1, f32x16 (&acc)[2][5]) {
  w8_read<MS>(f1, lds + (kt & 3) * P::STAGE, o, 32);
  sched_fence();
  w8_mma_loads<P, MS, LT, ISSUE_B ? 2 : 0>(f0, acc, rows, lds + ((kt + 2) & 3) * P::STAGE, (kt + 2) * P::BK * 2);
  if (WAIT >= 0) {
    wait_vm_only_barrier<(WAIT >= 0 ? WAIT : 0)>();
    w8_read<MS>(f0, lds + ((kt + 1) & 3) * P::STAGE, o, 0);
    sched_fence();
  }
  w8_mma_loads<P, MS, LT, ISSUE_A ? 1 : 0>(f1, acc, rows, lds + ((kt + 3) & 3) * P::STAGE, (kt + 3) * P::BK * 2);
}

// acc[j][i]: weight sub-tile j x token sub-tile i of this wave. K % 128 == 0
// (at least four stages). LT token load slots per stage (LT * 8 units cover
// the live rows).
template <class P, int MS, int LT>
__device__ __forceinline__ void w8_mainloop(const W8Rows& rows, int K, uint8_t* lds, const W8Offs& o,
                                            f32x16 (&acc)[2][5]) {
  static_assert(LT >= 1 && LT <= P::TLMAX && MS <= P::TT, "load slots");
  constexpr int LPS = P::WL + w8_min_token_loads<LT>();     // loads per stage of the waves with the fewest
  const int nk = K / P::BK;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
#pragma unroll
    for (int q = 0; q < P::WL; ++q) w8_issue_w<P>(rows, lds + s * P::STAGE, s * P::BK * 2, q);
    if (s < 2) {
#pragma unroll
      for (int q = 0; q < LT; ++q) w8_issue_t<P>(rows, lds + s * P::STAGE, s * P::BK * 2, q);
    }
  }
  wait_vm_only_barrier<LPS + P::WL>();                      // stage 0 complete (stage 1 and 2's weights may fly)
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0xc07f);                       // no scalar load pending: LDS waits stay partial
#endif
  W8Frags<MS> f0, f1;
  w8_read<MS>(f0, lds, o, 0);
  int kt = 0;
  for (; kt + 3 < nk; ++kt) w8_iteration<P, MS, LT, true, LPS, true>(rows, lds, kt, o, f0, f1, acc);
  w8_iteration<P, MS, LT, true, LPS, false>(rows, lds, kt, o, f0, f1, acc);        // kt = nk - 3
  w8_iteration<P, MS, LT, false, 0, false>(rows, lds, kt + 1, o, f0, f1, acc);     // kt = nk - 2
  w8_iteration<P, MS, LT, false, -1, false>(rows, lds, kt + 2, o, f0, f1, acc);    // kt = nk - 1
  // every wave has read the ring before the next tile's loads overwrite it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Live token sub-tiles of this wave (token half wt takes sub-tiles wt, wt + 2, ...) and token load slots.
__device__ __forceinline__ int w8_live(int nsub) { return (nsub + 1 - (threadIdx.x >> 8)) / 2; }

// Calls f(MS, LT) as compile-time constants for a block of nsub (1..10) sub-tiles.
#define W8_DISPATCH(nsub, CALL)                                                    \
  do {                                                                             \
    const int ms_ = w8_live(nsub), lt_ = ((nsub) + 3) / 4;                        \
    if (lt_ == 1) {                                                                \
      if (ms_ == 2) CALL(2, 1); else if (ms_ == 1) CALL(1, 1); else CALL(0, 1);   \
    } else if (lt_ == 2) {                                                         \
      if (ms_ == 4) CALL(4, 2); else if (ms_ == 3) CALL(3, 2); else CALL(2, 2);   \
    } else {                                                                       \
      if (ms_ == 5) CALL(5, 3); else CALL(4, 3);                                   \
    }                                                                              \
  } while (0)

// Token row (within the tile) of accumulator column l % 32 of token sub-tile i.
__device__ __forceinline__ int w8_token_row(int i, int tid) { return 32 * (2 * i + (tid >> 8)) + (tid & 31); }

}  // namespace moe
