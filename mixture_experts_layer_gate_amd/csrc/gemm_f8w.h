// Eight-wave pipelined E4M3 MFMA main loop with the scales applied per
// 128-wide K chunk, for the fp8 expert GEMMs at the large shapes
// ("DeepSeek_V3_Report: Annotation", sections "Fine-Grained Quantization" and
// "Increasing Accumulation Precision").
//
// The arithmetic is that of gemm_pipe8.h: output (w, n) is y = sum over chunks
// c of f_c * raw_c with f_c = s_token[n, c] * s_weight[block(w), c] and raw_c
// the chunk's E4M3 code dot product, accumulated by
// v_mfma_scale_f32_32x32x64_f8f6f4 in the frame of the current chunk
// (acc = partial sum / f_c) and moved to the next chunk's frame by one VALU
// multiply per element (r = f_c / f_{c+1}); factors below 1e-20 are raised to
// 1e-20.
//
// Tile: BW = 256 weight rows x BT = 256 token rows, eight waves (512 threads,
// two per SIMD). Wave w: weight half ww = w >> 2 (tile rows 128 ww .. +127:
// four 32-row sub-tiles j, for gate/up the gate sub-tiles 0, 1 and their up
// sub-tiles 2, 3, as in the tiled weight layout of moe_quantize_weights) and
// token quarter wt = w & 3 (sub-tiles wt and wt + 4): 4 x 2 accumulator tiles,
// 128 VGPRs, so two waves fit a SIMD. A token block of 256 rows lets a
// DeepSeek-V3 expert (256 rows on average) stream its weights once where the
// four-wave loop, with 128-row blocks, streamed them two or three times.
//
// Operands stream into LDS with buffer_load ... lds through a ring of four
// 32 KB stages of 64 K-bytes (one MFMA K step); rows of 64 bytes, 16-byte
// chunks XOR-swizzled by (row >> 2) & 3. Token scales come in windows of 8
// chunks: every 16 stages each thread loads four 4-byte scales of the next
// window into one of two LDS slots ([slot][row][8]), so K has no upper bound
// from a whole-K table. K must be a multiple of 1024 (whole windows).
//
// Iteration g (stage g of the unit's stream, chunk c = kt / 2 of its
// output-column block; f8w_stage gives the steps): the MFMAs of weight
// sub-tiles 0, 1; the barrier after stage g + 1 has landed; the reads of stage
// g + 1's sub-tiles 0, 1 and token fragments; the MFMAs of sub-tiles 2, 3 with
// the loads of stage g + 4 spread among them; the reads of stage g + 1's
// sub-tiles 2, 3; on a chunk's first stage the frame change. Each read is
// issued a group of MFMAs before its use (the token fragments double
// buffered), and the other wave of the SIMD covers the barrier waits. A tile
// moves to the next frame after its last MFMA of the chunk: sub-tiles 0, 1
// among the MFMAs of sub-tiles 2, 3 of the chunk's second stage, sub-tiles 2,
// 3 among the MFMAs of sub-tiles 0, 1 of the next chunk's first stage.
// A unit streams up to MAX_SEG output-column blocks that share its token rows
// as one sequence of stages.
#pragma once

#include "common.h"
#include "gemm_pipe.h"
#include "gemm_pipe8.h"

namespace moe {

struct F8W {
  static constexpr int BW = 256, BT = 256, BK = 64, NS = 4, NT = 512, NWAVE = 8;
  static constexpr int TW = 4, TT = 2;                     // 32x32 sub-tiles per wave
  static constexpr int MAXSUB = BT / 32;                   // token sub-tiles per block
  static constexpr int ROWB = BK;                          // bytes per row per stage
  static constexpr int W_BYTES = BW * ROWB, T_BYTES = BT * ROWB, STAGE = W_BYTES + T_BYTES;
  static constexpr int WL = W_BYTES / 16 / NT;             // weight loads per thread per stage (2)
  static constexpr int TL = T_BYTES / 16 / NT;             // token load slots per thread (2)
  static constexpr int RING = NS * STAGE;
  static constexpr int MAX_CHUNKS = 80;                    // weight-scale table: K <= 10240
  static constexpr int MAX_SEG = 4;                        // output-column blocks streamed per unit
  static constexpr int WIN = 8;                            // chunks per token-scale window
  static constexpr int SWL = BT * WIN / NT;                // window loads per thread (4)
  static constexpr int SW_OFF = RING;                      // weight scales [MAX_SEG][2][MAX_CHUNKS]
  static constexpr int SA_OFF = SW_OFF + MAX_SEG * 2 * MAX_CHUNKS * 4;   // token scales [2][BT][WIN]
  static constexpr int SRC_OFF = SA_OFF + 2 * BT * WIN * 4;              // source row of each tile row [BT]
  static constexpr int AMAX_OFF = SRC_OFF + BT * 4;                      // epilogue exchange [2][BT]
  static constexpr int LDS_BYTES = AMAX_OFF + 2 * BT * 4;
  static_assert(WL * NT * 16 == W_BYTES && TL * NT * 16 == T_BYTES, "stage must split evenly over the threads");
  static_assert(SWL * NT == BT * WIN, "window must split evenly over the threads");
};

// The workitem id, opaque to the optimizer: the per-lane offsets derived from
// it are then computed where they are used, inside the persistent unit loop,
// instead of being hoisted out of it and held in registers across the whole
// loop (which, next to 128 accumulators per lane, spills).
__device__ __forceinline__ int f8w_tid() {
  int t = threadIdx.x;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(t));
#endif
  return t;
}

// Wave coordinates and the output element of an accumulator.
struct F8WLayout {
  static constexpr int BW = F8W::BW, BT = F8W::BT, TW = F8W::TW, TT = F8W::TT;
  __device__ static int lane() { return f8w_tid() & 63; }
  __device__ static int ww() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 8); }
  __device__ static int wt() { return __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3); }
  // tile row of token sub-tile i of this lane
  __device__ static int token_row(int i) { return 32 * (4 * i + wt()) + (lane() & 31); }
  // output column (weight row within the tile) of accumulator elements 4q .. 4q+3 of weight sub-tile j
  __device__ static int wcol(int j, int q) { return ww() * 128 + j * 32 + 8 * q + 4 * (lane() >> 5); }
  // live token sub-tiles of this wave in a block of nsub
  __device__ static int live(int nsub) { return (wt() < nsub ? 1 : 0) + (wt() + 4 < nsub ? 1 : 0); }
};

struct F8WRows {
  __amdgpu_buffer_rsrc_t wrs, trs, srs;
  uint32_t ot[F8W::TL];    // token load slot q: source row * K + chunk * 16
  int kc;                  // K / 128: token scales per source row
};

// Token load slot q of this thread: 1 KB unit q * 8 + wave = tile rows 16 u .. 16 u + 15.
__device__ __forceinline__ int f8w_load_row(int q) { return (q * 8 + (threadIdx.x >> 6)) * 16 + ((threadIdx.x & 63) >> 2); }
__device__ __forceinline__ int f8w_load_chunk(int q) { return (threadIdx.x & 3) ^ ((f8w_load_row(q) >> 2) & 3); }
// Window load q of this thread: LDS float (q * 8 + wave) * 64 + lane of a slot = (row, chunk-in-window).
__device__ __forceinline__ int f8w_win_row(int q) { return ((q * 8 + (threadIdx.x >> 6)) * 64 + F8WLayout::lane()) >> 3; }
__device__ __forceinline__ int f8w_win_chunk() { return F8WLayout::lane() & 7; }

// Load q of stream stage s (segment-local K step ks) into its ring buffer:
// q < WL weights (stage s's 16 KB block, the unit's tiles being consecutive in
// the tiled layout), then token slot q - WL.
__device__ __forceinline__ void f8w_issue(const F8WRows& r, uint8_t* lds, int s, int ks, int q) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = F8W;
  uint8_t* st = lds + (s & 3) * P::STAGE;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (q < P::WL) {
    const uint32_t ow = static_cast<uint32_t>(((q * 8 + w) * 64 + F8WLayout::lane()) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.wrs, (lds_void_t*)(st + (q * 8 + w) * 1024), 16, ow, s * P::W_BYTES,
                                             0, 0);
  } else {
    const int qq = q - P::WL;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.trs, (lds_void_t*)(st + P::W_BYTES + (qq * 8 + w) * 1024), 16,
                                             r.ot[qq], ks * P::BK, 0, 0);
  }
#endif
}

// The token scales of window `win` (chunks 8 win .. 8 win + 7) of every tile row into slot `slot`; the
// rows' sources come from the unit's LDS table (its reads return before the loads issue).
__device__ __forceinline__ void f8w_issue_window(const F8WRows& r, uint8_t* lds, int slot, int win) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = F8W;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int* src = reinterpret_cast<const int*>(lds + P::SRC_OFF);
  uint32_t os[P::SWL];
#pragma unroll
  for (int q = 0; q < P::SWL; ++q) os[q] = (static_cast<uint32_t>(src[f8w_win_row(q)]) * r.kc + f8w_win_chunk()) * 4;
#pragma unroll
  for (int q = 0; q < P::SWL; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.srs, (lds_void_t*)(lds + P::SA_OFF + slot * P::BT * P::WIN * 4 +
                                                                  (q * 8 + w) * 256),
                                             4, os[q], win * P::WIN * 4, 0, 0);
#endif
}

// Per-lane byte offsets of the lane's two 16-byte pieces in a 32-row block of
// 64-byte stage rows (row l % 32, K bytes 32 (l / 32) .. +31 at their
// swizzled chunks): the same for every weight and token sub-tile.
struct F8WOffs {
  int lo, hi;
};
__device__ __forceinline__ F8WOffs f8w_offsets() {
  const int l = F8WLayout::lane(), sw = ((l & 31) >> 2) & 3, c0 = 2 * (l >> 5);
  return {(l & 31) * 64 + ((c0 ^ sw) << 4), (l & 31) * 64 + (((c0 + 1) ^ sw) << 4)};
}
__device__ __forceinline__ i32x8 f8w_frag(const uint8_t* base, const F8WOffs& o) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(base + o.lo);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(base + o.hi);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// Weight sub-tiles j0, j0 + 1 of this wave from stage buffer st.
__device__ __forceinline__ void f8w_read_w(i32x8 (&w)[F8W::TW], int j0, const uint8_t* st, const F8WOffs& o) {
  const uint8_t* b = st + F8WLayout::ww() * 128 * 64;
#pragma unroll
  for (int j = j0; j < j0 + 2; ++j) w[j] = f8w_frag(b + j * 32 * 64, o);
}
template <int MS>
__device__ __forceinline__ void f8w_read_t(i32x8 (&t)[F8W::TT], const uint8_t* st, const F8WOffs& o) {
  const uint8_t* b = st + F8W::W_BYTES + F8WLayout::wt() * 32 * 64;
#pragma unroll
  for (int i = 0; i < MS; ++i) t[i] = f8w_frag(b + i * 4 * 32 * 64, o);
}

// Weight-scale index of sub-tile j: gate/up tiles 0 (gate block) for j < 2,
// 1 (up block) otherwise; down tiles: the 128-row block of the wave's rows.
template <bool GATE_UP>
__device__ __forceinline__ int f8w_wb(int j) { return GATE_UP ? (j >= 2 ? 1 : 0) : 0; }
template <bool GATE_UP>
constexpr int f8w_nwb() { return GATE_UP ? 2 : 1; }

struct F8WFrame {
  float fac[2][F8W::TT];   // f of the current chunk per (weight-scale index, token sub-tile)
  float r[2][F8W::TT];     // f_c / f_{c+1}, or 1
};

__device__ __forceinline__ void f8w_scale_tile(f32x16& a, float r) {
#pragma unroll
  for (int v = 0; v < 16; ++v) a[v] *= r;
}

// The scales of chunk c of output-column block seg: token scales of this
// lane's rows from window slot `slot`, and the weight-block scale(s).
struct F8WScales {
  float sa[F8W::TT];
  float sw[2];
};
template <int MS, bool GATE_UP>
__device__ __forceinline__ void f8w_scale_loads(F8WScales& sc, const uint8_t* lds, int slot, int c, int seg) {
  const float* sat = reinterpret_cast<const float*>(lds + F8W::SA_OFF) + slot * F8W::BT * F8W::WIN + (c & 7);
  const float* swt = reinterpret_cast<const float*>(lds + F8W::SW_OFF) + seg * 2 * F8W::MAX_CHUNKS + c;
#pragma unroll
  for (int i = 0; i < MS; ++i) sc.sa[i] = sat[F8WLayout::token_row(i) * F8W::WIN];
  sc.sw[0] = swt[(GATE_UP ? 0 : F8WLayout::ww()) * F8W::MAX_CHUNKS];
  if (GATE_UP) sc.sw[1] = swt[F8W::MAX_CHUNKS];
}
// fac := factors of the scales in sc (r := fac_old / fac_new when `next`, else 1).
template <int MS, bool GATE_UP>
__device__ __forceinline__ void f8w_frame_update(F8WFrame& fr, const F8WScales& sc, bool next,
                                                 bool first) {
#pragma unroll
  for (int b = 0; b < f8w_nwb<GATE_UP>(); ++b)
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const float fn = fmaxf(sc.sa[i] * sc.sw[b], kMinFactor);
      fr.r[b][i] = (next && !first) ? fr.fac[b][i] * __builtin_amdgcn_rcpf(fn) : 1.0f;
      fr.fac[b][i] = fn;
    }
}

// The MFMAs of weight sub-tiles 0, 1 (tile m = (m / MS, m % MS)). FIRST (a
// chunk's first stage): sub-tile 2, 3 tile m moves to this chunk's frame right
// before MFMA m.
template <int MS, bool GATE_UP, bool FIRST>
__device__ __forceinline__ void f8w_mma_lo(const i32x8 (&w)[F8W::TW], const i32x8 (&t)[F8W::TT],
                                           f32x16 (&acc)[F8W::TW][F8W::TT], const F8WFrame& fr) {
  constexpr int M = 2 * MS, D = MS > 0 ? MS : 1;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (FIRST) f8w_scale_tile(acc[2 + m / D][m % D], fr.r[f8w_wb<GATE_UP>(2)][m % D]);
    acc[m / D][m % D] = mfma_f8(w[m / D], t[m % D], acc[m / D][m % D]);
    sched_fence();
  }
  sched_fence();
}

// The MFMAs of weight sub-tiles 2, 3 (tile m = (2 + m / MS, m % MS)) with
// L = WL + LT loads of stage ls spread among them (load q before MFMA
// q * M / L) when ISSUE. SECOND (a chunk's second stage): sub-tile 0, 1 tile m
// moves to the next frame right after MFMA m (its last MFMA of the chunk was
// before the barrier).
template <int MS, int LT, bool GATE_UP, bool SECOND, bool ISSUE>
__device__ __forceinline__ void f8w_mma_hi(const i32x8 (&w)[F8W::TW], const i32x8 (&t)[F8W::TT],
                                           f32x16 (&acc)[F8W::TW][F8W::TT], const F8WFrame& fr,
                                           const F8WRows& rows, uint8_t* lds, int ls, int lks) {
  constexpr int M = 2 * MS, D = MS > 0 ? MS : 1;
  constexpr int L = ISSUE ? F8W::WL + LT : 0;
#pragma unroll
  for (int n = 0; n < (M > L ? M : L); ++n) {
#pragma unroll
    for (int q = 0; q < L; ++q)
      if ((M == 0 && q == n) || (M > 0 && q * M / (L > 0 ? L : 1) == n)) {
        f8w_issue(rows, lds, ls, lks, q);
        sched_fence();
      }
    if (n < M) {
      acc[2 + n / D][n % D] = mfma_f8(w[2 + n / D], t[n % D], acc[2 + n / D][n % D]);
      if (SECOND) f8w_scale_tile(acc[n / D][n % D], fr.r[f8w_wb<GATE_UP>(0)][n % D]);
      sched_fence();
    }
  }
  sched_fence();
}

// One stage of the stream (global index g, segment-local kt, chunk kt / 2 of
// output-column block seg): w holds its weight fragments, T0 its token
// fragments; w and T1 receive stage g + 1's.
//   a. the MFMAs of weight sub-tiles 0, 1;
//   b. wait until stage g + 1 has landed and every LDS read of this wave has
//      returned, barrier; every 8 chunks (a chunk's first stage) the loads of
//      the next token-scale window;
//   c. read stage g + 1's weight sub-tiles 0, 1 and token sub-tiles into w,
//      T1; the MFMAs of weight sub-tiles 2, 3 with the loads of stage g + 4
//      spread among them (into the buffer of stage g, whose reads all returned
//      before the barrier);
//   d. read stage g + 1's weight sub-tiles 2, 3;
//   e. (a chunk's first stage) the scales of chunk c + 1 and the frame change
//      r = f_c / f_{c+1}.
// Each read is issued a group of MFMAs before its fragments are used, so its
// latency is covered. WAIT: loads allowed in flight at the barrier (those of
// the stages after g + 1 that exist), or -1 for the stream's last stage (no
// barrier, nothing to read). ISSUE: load stage g + 4.
template <int MS, int LT, bool GATE_UP, bool SECOND, int WAIT, bool ISSUE>
__device__ __forceinline__ void f8w_stage(const F8WRows& rows, uint8_t* lds, const F8WOffs& o, int g, int kt, int nk,
                                          int kc, int seg, int nseg, i32x8 (&w)[F8W::TW],
                                          const i32x8 (&T0)[F8W::TT], i32x8 (&T1)[F8W::TT],
                                          f32x16 (&acc)[F8W::TW][F8W::TT], F8WFrame& fr) {
  using P = F8W;
  const int c = kt >> 1, nwin = kc / P::WIN, gw = seg * nwin + (c >> 3);
  f8w_mma_lo<MS, GATE_UP, !SECOND>(w, T0, acc, fr);
  if (WAIT >= 0) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(WAIT >= 0 ? WAIT : 0) : "memory");
    if (!SECOND && (c & 7) == 0) {
      // the next token-scale window: this block's, else the next block's first
      if ((c >> 3) + 1 < nwin) f8w_issue_window(rows, lds, (gw + 1) & 1, (c >> 3) + 1);
      else if (seg + 1 < nseg) f8w_issue_window(rows, lds, (gw + 1) & 1, 0);
      sched_fence();
    }
    const uint8_t* st = lds + ((g + 1) & 3) * P::STAGE;
    f8w_read_w(w, 0, st, o);
    f8w_read_t<MS>(T1, st, o);
    sched_fence();
  }
  int ks4 = kt + 4;
  if (ks4 >= nk) ks4 -= nk;
  f8w_mma_hi<MS, LT, GATE_UP, SECOND, ISSUE>(w, T0, acc, fr, rows, lds, g + 4, ks4);
  if (WAIT >= 0) {
    f8w_read_w(w, 2, lds + ((g + 1) & 3) * P::STAGE, o);
    sched_fence();
  }
  if (!SECOND) {
    const bool next = c + 1 < kc;
    const int cn = next ? c + 1 : c;
    F8WScales sc;
    f8w_scale_loads<MS, GATE_UP>(sc, lds, (seg * nwin + (cn >> 3)) & 1, cn, seg);
    f8w_frame_update<MS, GATE_UP>(fr, sc, next, false);
  }
}

// End of output-column block seg: y = acc * (last chunk's factor) for the
// epilogue, then acc restarts from zero in the frame of the next block's
// first chunk (its window landed with the stages since it was issued).
template <int MS, bool GATE_UP, class EPI>
__device__ __forceinline__ void f8w_finish(f32x16 (&acc)[F8W::TW][F8W::TT], F8WFrame& fr, EPI& epi,
                                           int seg, int nseg, int kc, const uint8_t* lds) {
#pragma unroll
  for (int j = 0; j < F8W::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i) f8w_scale_tile(acc[j][i], fr.fac[f8w_wb<GATE_UP>(j)][i]);
  epi(seg, acc);
#pragma unroll
  for (int j = 0; j < F8W::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  if (seg + 1 < nseg) {
    F8WScales sc;
    f8w_scale_loads<MS, GATE_UP>(sc, lds, ((seg + 1) * (kc / F8W::WIN)) & 1, 0, seg + 1);
    f8w_frame_update<MS, GATE_UP>(fr, sc, false, true);
  }
}

// The K loops of nseg output-column blocks of one unit as one stream of
// S = nseg * nk stages through the ring. For each block: acc = the block's
// outputs, then epi(seg, acc) (stores; may use AMAX_OFF with LDS-only
// barriers). K % 1024 == 0, K / 128 <= MAX_CHUNKS, nseg <= MAX_SEG. Before the
// call the unit's weight scales ([seg][2][chunk]) are in LDS and visible to
// every wave. LT (>= 1) token load slots per stage cover the live rows.
template <int MS, int LT, bool GATE_UP, class EPI>
__device__ __forceinline__ void f8w_stream(const F8WRows& rows, int K, int nseg, uint8_t* lds, EPI& epi) {
  using P = F8W;
  static_assert(LT >= 1 && LT <= P::TL && MS <= P::TT, "token load slots");
  constexpr int LPS = P::WL + LT;                      // loads per stage per thread
  static_assert(3 * LPS + P::SWL <= 63, "vmcnt range");
  const int nk = K / P::BK, kc = K / 128, S = nseg * nk;   // nk >= 16, S >= 16
  f8w_issue_window(rows, lds, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int q = 0; q < LPS; ++q) f8w_issue(rows, lds, s, s, q);
  }
  // window 0 and stage 0 have landed
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(3 * LPS) : "memory");
  const F8WOffs o = f8w_offsets();
  f32x16 acc[P::TW][P::TT];
  F8WFrame fr;
#pragma unroll
  for (int j = 0; j < P::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  {
    F8WScales sc;
    f8w_scale_loads<MS, GATE_UP>(sc, lds, 0, 0, 0);
    f8w_frame_update<MS, GATE_UP>(fr, sc, false, true);
  }
  i32x8 w[P::TW], T0[P::TT], T1[P::TT];
  f8w_read_w(w, 0, lds, o);
  f8w_read_t<MS>(T0, lds, o);
  f8w_read_w(w, 2, lds, o);
  int g = 0, kt = 0, seg = 0;
  for (; g + 6 <= S; g += 2) {                         // both stages refill the ring
    f8w_stage<MS, LT, GATE_UP, false, 2 * LPS, true>(rows, lds, o, g, kt, nk, kc, seg, nseg, w, T0, T1, acc, fr);
    f8w_stage<MS, LT, GATE_UP, true, 2 * LPS, true>(rows, lds, o, g + 1, kt + 1, nk, kc, seg, nseg, w, T1, T0, acc,
                                                    fr);
    kt += 2;
    if (kt == nk) {
      f8w_finish<MS, GATE_UP>(acc, fr, epi, seg, nseg, kc, lds);
      ++seg;
      kt = 0;
    }
  }
  // S - g == 4, all in the last block: the stream's last four stages load nothing
  f8w_stage<MS, LT, GATE_UP, false, 2 * LPS, false>(rows, lds, o, g, kt, nk, kc, seg, nseg, w, T0, T1, acc, fr);
  f8w_stage<MS, LT, GATE_UP, true, LPS, false>(rows, lds, o, g + 1, kt + 1, nk, kc, seg, nseg, w, T1, T0, acc, fr);
  f8w_stage<MS, LT, GATE_UP, false, 0, false>(rows, lds, o, g + 2, kt + 2, nk, kc, seg, nseg, w, T0, T1, acc, fr);
  f8w_stage<MS, LT, GATE_UP, true, -1, false>(rows, lds, o, g + 3, kt + 3, nk, kc, seg, nseg, w, T1, T0, acc, fr);
  f8w_finish<MS, GATE_UP>(acc, fr, epi, seg, nseg, kc, lds);
  // every wave has read the ring and the tables before the next unit overwrites them
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe
