// Pipelined bf16 MFMA main loop for the expert GEMMs.
//
// Tile: BW weight rows x BT token rows, K-contiguous bf16 operands. The
// weight rows are the MFMA's first operand, so each lane's accumulator holds
// four consecutive output columns of one token row (8-byte stores).
//
// Both operands stream from global memory straight into LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging) through a ring of NS = 4 stages of
// BK = 32 K-elements; up to three stages are in flight while one is consumed
// (about 96 KB per CU outstanding, enough to cover HBM latency at full rate). Four
// waves in a 2 x 2 grid each own a 128 x 128 block of 32x32x16 MFMA sub-tiles,
// so every LDS fragment feeds four MFMAs. The two wave rows take the token
// sub-tiles round-robin (wave row wt: sub-tiles wt, wt+2, ...), and only the
// MS (compile time) live ones are computed.
//
// Schedule of one stage (two K16 steps) per wave: read step-1 fragments;
// 16 MFMAs on step-0 fragments; wait for the next stage's loads + barrier;
// issue the loads three stages ahead (into the buffer every wave has finished
// with); read the next stage's step-0 fragments; 16 MFMAs on the step-1
// fragments. The barrier needs no LDS read to be complete (see pipe_mainloop).
//
// LDS layout per stage: rows of 64 bytes (4 chunks of 16 B). A direct load
// writes 64 consecutive chunks, one per lane; chunk p holds row p / 4 and
// logical K chunk (p % 4) ^ ((row >> 2) & 3). The XOR spreads the eight
// lanes the LDS serves together (rows r .. r+7 at one logical chunk) over
// eight bank groups.
//
// Synchronisation uses s_waitcnt + s_barrier in one asm statement with a
// memory clobber: the barrier builtin alone is not a memory barrier to the
// compiler, and the compiler does not track the LDS writes of the DMA loads.
#pragma once

#include "common.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;

// TILED: the weight rows come in the tiled layout of moe_tile_weights_bf16 (a
// tile's 32-wide K steps are contiguous 16 KB blocks that are the stages' LDS
// images); weight load q of a thread then reads the 16 bytes at
// ((q * 4 + wave) * 64 + lane) * 16 of the block of K step kb / 64.
template <int BW_, int BT_, bool TILED_ = false>
struct Pipe {
  static constexpr int BW = BW_, BT = BT_, BK = 32, NS = 4, NT = 256;
  static constexpr bool TILED = TILED_;
  static constexpr int TW = BW / 64, TT = BT / 64;          // 32x32 sub-tiles per wave
  static constexpr int ROWB = BK * 2;                        // bytes per row per stage
  static constexpr int W_BYTES = BW * ROWB, T_BYTES = BT * ROWB, STAGE = W_BYTES + T_BYTES;
  static constexpr int WL = W_BYTES / 16 / NT, TL = T_BYTES / 16 / NT;  // loads per thread per stage
  static constexpr int LPS = WL + TL;
  static constexpr int LDS_BYTES = NS * STAGE;
  static_assert(WL * NT * 16 == W_BYTES && TL * NT * 16 == T_BYTES, "stage must split evenly over the threads");
  static_assert(LPS * 3 <= 63, "vmcnt range");
};

// Tile row and logical K chunk (16 B) of load q of this thread.
__device__ __forceinline__ int pipe_load_row(int q) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  return (q * 4 + w) * 16 + (l >> 2);
}
__device__ __forceinline__ int pipe_load_chunk(int q) {
  const int l = threadIdx.x & 63;
  return (l & 3) ^ ((pipe_load_row(q) >> 2) & 3);
}

// Operand rows of this thread as buffer resources (wave-uniform base and size
// in bytes) plus 32-bit byte offsets (row * K * 2 + logical chunk * 16). The
// MUBUF form of the LDS-DMA load takes the stage's K offset in an SGPR, so a
// load costs no address arithmetic; unlike the FLAT form it also leaves the
// compiler's LDS-counter model in order, so fragment waits stay partial.
template <class P>
struct PipeRows {
  __amdgpu_buffer_rsrc_t wrs, trs;
  uint32_t ow[P::WL];
  uint32_t ot[P::TL];
};

// Buffer resource over [base, base + bytes); bytes must be below 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pipe_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                          static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
}

// Part A of a stage = its weight rows (WL loads per thread), part B = its
// token rows (TL loads per thread). Load q of a part goes to LDS chunk block
// q * 4 + wave (1 KB each).
template <class P, bool A>
__device__ __forceinline__ void pipe_issue_one(const PipeRows<P>& r, uint8_t* st, int kb, int q) {
#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-DMA builtin exists only in the device pass
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS address in SGPRs
  if (A)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.wrs, (lds_void_t*)(st + (q * 4 + w) * 1024), 16, r.ow[q],
                                             P::TILED ? kb * (P::W_BYTES / P::ROWB) : kb, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.trs, (lds_void_t*)(st + P::W_BYTES + (q * 4 + w) * 1024), 16, r.ot[q],
                                             kb, 0, 0);
#endif
}

// LT: token load groups issued per stage (group q covers tile rows 64q .. 64q+63);
// blocks with fewer live rows skip the groups past them.
template <class P, bool A, int LT>
__device__ __forceinline__ void pipe_issue_part(const PipeRows<P>& r, uint8_t* lds, int stage, int k0) {
#pragma unroll
  for (int q = 0; q < (A ? P::WL : LT); ++q) pipe_issue_one<P, A>(r, lds + stage * P::STAGE, k0 * 2, q);
}

template <class P, int MS>
struct PipeFrags {
  bf16x8 w[P::TW];
  bf16x8 t[MS > 0 ? MS : 1];
};

// Token sub-tile i of this wave: tile rows 32 * (2 i + wt) .. +31.
template <class P, int MS>
__device__ __forceinline__ void pipe_read(PipeFrags<P, MS>& f, const uint8_t* st, int w_off, int t_off, int flip) {
#pragma unroll
  for (int j = 0; j < P::TW; ++j) f.w[j] = *reinterpret_cast<const bf16x8*>(st + ((w_off + j * 32 * P::ROWB) ^ flip));
#pragma unroll
  for (int i = 0; i < MS; ++i)
    f.t[i] = *reinterpret_cast<const bf16x8*>(st + ((t_off + i * 64 * P::ROWB) ^ flip));
}

template <class P, int MS>
__device__ __forceinline__ void pipe_mma(const PipeFrags<P, MS>& f, f32x16 (&acc)[P::TW][P::TT]) {
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < P::TW; ++j) acc[j][i] = mfma_32x32x16_bf16(f.w[j], f.t[i], acc[j][i]);
}

// Keeps the scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// The MFMAs of one K16 step with one part of a stage's loads spread evenly
// among them (load q before MFMA q * M / L), so the vector-memory pipe is fed
// steadily: issued as one burst, the loads back up and the wave, which issues
// in order, stalls with its MFMAs behind them.
template <class P, int MS, int LT, int PART>  // PART: 0 none, 1 part A, 2 part B
__device__ __forceinline__ void pipe_mma_loads(const PipeFrags<P, MS>& f, f32x16 (&acc)[P::TW][P::TT],
                                               const PipeRows<P>& r, uint8_t* st, int kb) {
  constexpr int M = P::TW * MS;
  constexpr int L = PART == 0 ? 0 : (PART == 1 ? P::WL : LT);
#pragma unroll
  for (int m = 0; m < (M > L ? M : L); ++m) {
#pragma unroll
    for (int q = 0; q < L; ++q)
      if ((M == 0 && q == m) || (M > 0 && q * M / (L > 0 ? L : 1) == m)) {
        pipe_issue_one<P, PART == 1>(r, st, kb, q);
        sched_fence();
      }
    if (m < M) acc[m % P::TW][m / P::TW] = mfma_32x32x16_bf16(f.w[m % P::TW], f.t[m / P::TW], acc[m % P::TW][m / P::TW]);
  }
  sched_fence();
}

template <int N>
__device__ __forceinline__ void wait_vm_only_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One stage kt (two K16 steps) per wave. Stage s is issued in two parts: part
// A (weights) among the step-1 MFMAs of iteration s - 3, part B (tokens) among
// the step-0 MFMAs of iteration s - 2; both follow the barrier of iteration
// s - 3, after which every wave has finished reading the buffer s % 4 (it last
// held stage s - 4, read for iteration s - 4). At the barrier of iteration kt
// only stage kt + 2 may still be in flight (LPS loads), so stage kt + 1 is
// complete. The barrier needs no LDS read to be complete.
//   ISSUE_B: issue part B of stage kt + 2; WAIT: vmcnt at the barrier, or -1
//   for no barrier (last stage); ISSUE_A: issue part A of stage kt + 3.
template <class P, int MS, int LT, bool ISSUE_B, int WAIT, bool ISSUE_A>
__device__ __forceinline__ void pipe_iteration(const PipeRows<P>& rows, uint8_t* lds, int kt, int w_off, int t_off,
                                               PipeFrags<P, MS>& f0, PipeFrags<P, MS>& f1,
                                               f32x16 (&acc)[P::TW][P::TT]) {
  pipe_read<P, MS>(f1, lds + (kt & 3) * P::STAGE, w_off, t_off, 32);
  sched_fence();
  pipe_mma_loads<P, MS, LT, ISSUE_B ? 2 : 0>(f0, acc, rows, lds + ((kt + 2) & 3) * P::STAGE, (kt + 2) * P::BK * 2);
  if (WAIT >= 0) {
    wait_vm_only_barrier<(WAIT >= 0 ? WAIT : 0)>();
    pipe_read<P, MS>(f0, lds + ((kt + 1) & 3) * P::STAGE, w_off, t_off, 0);
    sched_fence();
  }
  pipe_mma_loads<P, MS, LT, ISSUE_A ? 1 : 0>(f1, acc, rows, lds + ((kt + 3) & 3) * P::STAGE, (kt + 3) * P::BK * 2);
}

// acc[j][i]: weight sub-tile j x token sub-tile i of this wave. K % 128 == 0,
// so there are at least four stages. LT (>= MS of every wave) token load
// groups per stage.
template <class P, int MS, int LT>
__device__ __forceinline__ void pipe_mainloop(const PipeRows<P>& rows, int K, uint8_t* lds,
                                              f32x16 (&acc)[P::TW][P::TT]) {
  static_assert(P::NS == 4, "schedule written for a ring of four stages");
  static_assert(LT >= 1 && LT <= P::TL && 2 * LT >= 2 * MS, "token load groups must cover the live sub-tiles");
  constexpr int LPS = P::WL + LT;                           // loads per stage per thread
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wt = w & 1, ww = w >> 1;
  const int nk = K / P::BK;
  const int sw = ((l & 31) >> 2) & 3;
  const int cofs = ((l >> 5) ^ sw) * 16;                    // step 0; step 1 flips bit 5
  const int w_off = (ww * (P::BW / 2) + (l & 31)) * P::ROWB + cofs;
  const int t_off = P::W_BYTES + (wt * 32 + (l & 31)) * P::ROWB + cofs;

  pipe_issue_part<P, true, LT>(rows, lds, 0, 0);
  pipe_issue_part<P, false, LT>(rows, lds, 0, 0);
  pipe_issue_part<P, true, LT>(rows, lds, 1, P::BK);
  pipe_issue_part<P, false, LT>(rows, lds, 1, P::BK);
  pipe_issue_part<P, true, LT>(rows, lds, 2, 2 * P::BK);
  wait_vm_only_barrier<LPS + P::WL>();                      // stage 0 complete
#if defined(__HIP_DEVICE_COMPILE__)
  // Retire any scalar load still in flight (lgkmcnt(0), other counters left
  // free) in a form the compiler sees: with none pending, the LDS counter
  // stays in order inside the loop and fragment waits can be partial.
  __builtin_amdgcn_s_waitcnt(0xc07f);
#endif

  PipeFrags<P, MS> f0, f1;
  pipe_read<P, MS>(f0, lds, w_off, t_off, 0);
  int kt = 0;
  for (; kt + 3 < nk; ++kt) pipe_iteration<P, MS, LT, true, LPS, true>(rows, lds, kt, w_off, t_off, f0, f1, acc);
  pipe_iteration<P, MS, LT, true, LPS, false>(rows, lds, kt, w_off, t_off, f0, f1, acc);     // kt = nk - 3
  pipe_iteration<P, MS, LT, false, 0, false>(rows, lds, kt + 1, w_off, t_off, f0, f1, acc);  // kt = nk - 2
  pipe_iteration<P, MS, LT, false, -1, false>(rows, lds, kt + 2, w_off, t_off, f0, f1, acc); // kt = nk - 1
  // every wave has read the ring before the next tile's loads overwrite it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Accumulator element v of sub-tile (j, i): tile token row, and the first of
// the four consecutive tile weight rows (output columns) held in v = 4q .. 4q+3.
__device__ __forceinline__ int pipe_token_row(int i) {
  const int l = threadIdx.x & 63, wt = (threadIdx.x >> 6) & 1;
  return 32 * (2 * i + wt) + (l & 31);
}
template <class P>
__device__ __forceinline__ int pipe_wcol(int j, int q) {
  const int l = threadIdx.x & 63, ww = threadIdx.x >> 7;
  return ww * (P::BW / 2) + j * 32 + 8 * q + 4 * (l >> 5);
}

}  // namespace moe
