// bf16 MFMA main loop: a BM x BN fp32 tile of A . B^T over K, both operands
// K-contiguous bf16 rows, staged through double-buffered LDS.
//
// Each thread owns AC (resp. BC) 16-byte chunks of the A (B) tile: chunk
// c = tid + NT*j covers row c/8, columns 8*(c%8) .. +7 of a BK = 64 slice, so
// eight consecutive threads read one 128-byte row segment. A null row
// pointer reads zeros (rows past the end of a ragged expert segment).
// LDS rows are padded to 72 elements (144 B) so the 32 rows touched by one
// MFMA operand read fall in distinct banks.
#pragma once

#include "common.h"

namespace moe {

template <int BM_, int BN_, int WM_, int WN_>
struct TileBF16 {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = 64;
  static constexpr int LDK = BK + 8;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int TM = BM / (32 * WM);
  static constexpr int TN = BN / (32 * WN);
  static constexpr int AC = BM * (BK / 8) / NT;
  static constexpr int BC = BN * (BK / 8) / NT;
  static constexpr int LDS_BYTES = 2 * (BM + BN) * LDK * 2;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  static_assert(AC >= 1 && BC >= 1 && AC * NT == BM * (BK / 8) && BC * NT == BN * (BK / 8),
                "tile chunks must divide evenly over the threads");
};

// Row index (within the tile) of chunk j of thread tid.
template <class G>
__device__ __forceinline__ int chunk_row(int tid, int j) { return (tid + G::NT * j) >> 3; }
template <class G>
__device__ __forceinline__ int chunk_col(int tid, int j) { return ((tid + G::NT * j) & 7) * 8; }

template <class G>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[G::TM][G::TN]) {
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
}

// acc += A . B^T over K (a multiple of 64). pa / pb: this thread's row
// pointers (already offset by its chunk column), or nullptr for zero rows.
template <class G>
__device__ __forceinline__ void mainloop_bf16(const uint16_t* const (&pa)[G::AC],
                                              const uint16_t* const (&pb)[G::BC], int K,
                                              uint16_t* lds, f32x16 (&acc)[G::TM][G::TN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % G::WM;
  const int wn = wave / G::WM;
  uint16_t* As = lds;                              // [2][BM][LDK]
  uint16_t* Bs = lds + 2 * G::BM * G::LDK;         // [2][BN][LDK]
  u32x4 ra[G::AC], rb[G::BC];
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int nk = K / G::BK;

#pragma unroll
  for (int j = 0; j < G::AC; ++j) ra[j] = pa[j] ? *reinterpret_cast<const u32x4*>(pa[j]) : z;
#pragma unroll
  for (int j = 0; j < G::BC; ++j) rb[j] = pb[j] ? *reinterpret_cast<const u32x4*>(pb[j]) : z;
#pragma unroll
  for (int j = 0; j < G::AC; ++j)
    *reinterpret_cast<u32x4*>(&As[chunk_row<G>(tid, j) * G::LDK + chunk_col<G>(tid, j)]) = ra[j];
#pragma unroll
  for (int j = 0; j < G::BC; ++j)
    *reinterpret_cast<u32x4*>(&Bs[chunk_row<G>(tid, j) * G::LDK + chunk_col<G>(tid, j)]) = rb[j];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = (kt + 1) * G::BK;
#pragma unroll
      for (int j = 0; j < G::AC; ++j) ra[j] = pa[j] ? *reinterpret_cast<const u32x4*>(pa[j] + k0) : z;
#pragma unroll
      for (int j = 0; j < G::BC; ++j) rb[j] = pb[j] ? *reinterpret_cast<const u32x4*>(pb[j] + k0) : z;
    }
    const uint16_t* Ab = As + buf * G::BM * G::LDK;
    const uint16_t* Bb = Bs + buf * G::BN * G::LDK;
#pragma unroll
    for (int s = 0; s < G::BK / 16; ++s) {
      const int kof = s * 16 + 8 * (lane >> 5);
      bf16x8 af[G::TM], bf[G::TN];
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&Ab[(wm * G::TM * 32 + i * 32 + (lane & 31)) * G::LDK + kof]);
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(&Bb[(wn * G::TN * 32 + j * 32 + (lane & 31)) * G::LDK + kof]);
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = mfma_32x32x16_bf16(af[i], bf[j], acc[i][j]);
    }
    if (more) {
      uint16_t* An = As + (buf ^ 1) * G::BM * G::LDK;
      uint16_t* Bn = Bs + (buf ^ 1) * G::BN * G::LDK;
#pragma unroll
      for (int j = 0; j < G::AC; ++j)
        *reinterpret_cast<u32x4*>(&An[chunk_row<G>(tid, j) * G::LDK + chunk_col<G>(tid, j)]) = ra[j];
#pragma unroll
      for (int j = 0; j < G::BC; ++j)
        *reinterpret_cast<u32x4*>(&Bn[chunk_row<G>(tid, j) * G::LDK + chunk_col<G>(tid, j)]) = rb[j];
    }
    __syncthreads();
  }
}

// Tile-local (row, col) of accumulator element v of sub-tile (i, j) for this lane.
template <class G>
__device__ __forceinline__ int acc_row(int i, int v) {
  const int lane = threadIdx.x & 63;
  const int wm = (threadIdx.x >> 6) % G::WM;
  return wm * G::TM * 32 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
template <class G>
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63;
  const int wn = (threadIdx.x >> 6) / G::WM;
  return wn * G::TN * 32 + j * 32 + (lane & 31);
}

}  // namespace moe
