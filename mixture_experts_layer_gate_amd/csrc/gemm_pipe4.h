// Pipelined MFMA main loop for MXFP4 expert weights times E4M3 activations
// ("DeepSeek V3 / V4 Infra", V4 post-training FP4 QAT of the expert weights;
// the activations keep the V3 fp8 recipe of "DeepSeek_V3_Report: Annotation",
// section "Fine-Grained Quantization").
//
// Weights are E2M1 codes (two per byte, the even K index in the low nibble)
// with one E8M0 scale per 32 consecutive K values; tokens are E4M3 codes with
// one fp32 scale per 1x128 tile. gfx950's v_mfma_scale_f32_32x32x64_f8f6f4
// reads an E2M1 first operand and applies a per-lane E8M0 scale to it: lane l
// holds weight row l % 32 at K 32 (l / 32) .. +31 (16 bytes) and supplies the
// scale of exactly that 32-value block, so the weights' scales cost nothing
// beyond a byte per lane and MFMA. (Its E4M3 second operand interleaves K:
// lane half h holds K 16h .. 16h+15 in bytes 0..15 and K 32+16h .. 32+16h+15
// in bytes 16..31.) The token scales are fp32 and stay on the VALU: the
// accumulator is kept in the frame of the current 128-wide chunk as in
// gemm_pipe8.h, acc = (sum over chunks c' <= c of s_c' raw_c') / s_c with s_c
// the token's scale, rescaled by s_c / s_{c+1} between chunks and by the last
// s at the end; factors below 1e-20 are raised to 1e-20.
//
// Tile: BW = 256 weight rows x BT = 128 token rows, four waves in a 2 x 2 grid
// of 128 x 64, as in gemm_pipe8.h. A stage covers 64 K values: 32-byte weight
// rows and 64-byte token rows, streamed into LDS with buffer_load ... lds
// through a ring of seven stages (a stage holds half the weight bytes of an
// E4M3 stage; up to five are in flight while one is consumed: a CU's load
// throughput is its bytes in flight over the memory latency, and the decode
// batch streams little besides the weights). The weights come in
// the tiled layout of moe_quantize_weights_mxfp4: a tile's 8 KB of codes per
// stage are one contiguous block that is already the stage's LDS image (rows
// of 32 bytes, 16-byte halves XOR-swizzled), and its weight scales per chunk
// (two stages: four 32-value blocks x 256 rows) one contiguous 1 KB block, so
// every load instruction reads 1 KB of consecutive bytes and the stages of a
// unit's column blocks follow each other in memory. The chunk's scales come in
// one 16-byte-per-lane load of wave 0, issued just before the chunk's first
// stage, into a ring of four chunk slots; wave 0 therefore counts one more
// load per chunk than the other waves, and its waits allow for it.
#pragma once

#include "common.h"
#include "gemm_pipe.h"
#include "gemm_pipe8.h"

namespace moe {

struct Pipe4 {
  static constexpr int BW = 256, BT = 128, BK = 64, NS = 7, NT = 256, NWAVE = NT / 64;
  static constexpr int TW = 4, TT = 2;                    // 32x32 sub-tiles per wave
  static constexpr int WROWB = BK / 2, TROWB = BK;         // bytes per row per stage
  static constexpr int W_BYTES = BW * WROWB;               // E2M1 codes
  static constexpr int T_BYTES = BT * TROWB;               // E4M3 codes
  static constexpr int T_OFF = W_BYTES;
  static constexpr int STAGE = W_BYTES + T_BYTES;
  static constexpr int WL = W_BYTES / 16 / NT, TL = T_BYTES / 16 / NT;
  static constexpr int RING = NS * STAGE;
  static constexpr int SC_SLOTS = 4, SC_BYTES = 4 * BW;    // chunk slots of [K block][row] E8M0 scales
  static constexpr int SC_OFF = RING;
  static constexpr int MAX_CHUNKS = 64;                    // K <= 8192
  static constexpr int MAX_SEG = 2;                        // output-column blocks streamed per unit (*)
  static constexpr int SA_OFF = SC_OFF + SC_SLOTS * SC_BYTES;    // token scales [BT][kc_pad]
  static constexpr int SRC_OFF = SA_OFF + BT * MAX_CHUNKS * 4;   // source row of each tile row [BT]
  static constexpr int AMAX_OFF = SRC_OFF + BT * 4;              // epilogue exchange [2][BT]
  static constexpr int LDS_BYTES = AMAX_OFF + 2 * BT * 4;
  static_assert(WL * NT * 16 == W_BYTES && TL * NT * 16 == T_BYTES, "stage must split evenly over the threads");
  static_assert(64 * 16 == SC_BYTES, "one wave's 16-byte load covers a chunk's scales");
  static_assert((WL + TL) * (NS - 2) + 2 <= 63, "vmcnt range");
  // (*) Units of two column blocks balance the CUs better than four: decode batch gate/up 1.25 -> 1.20 ms,
  // down 0.63 -> 0.615 ms; V3 gate/up 3.02-3.05 -> 2.98 ms (one block: 1.22 / 0.66 and 2.98 / 1.77 ms).
  static_assert(BW == Pipe8::BW && BT == Pipe8::BT && TW == Pipe8::TW && TT == Pipe8::TT,
                "same tile and wave layout as the E4M3 loop (shared epilogues)");
};

__device__ __forceinline__ int p4_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Operand resources: the unit's weight codes and scales from its first
// column block on (the stream's stages and chunks are consecutive blocks of
// 8 KB and 1 KB), and the token codes with per-thread 32-bit row offsets (as
// gemm_pipe8.h). Weight load q of this thread reads the 16 bytes at
// ((q * NWAVE + wave) * 64 + lane) * 16 of the stage's block, the scale load
// (wave 0) the 16 bytes at lane * 16 of the chunk's block: the LDS images.
struct Pipe4Rows {
  __amdgpu_buffer_rsrc_t wrs, srs, trs;
  uint32_t ot[Pipe4::TL];
};

// Stage s of the stream (output-column block seg = s / nk, local stage ks):
// its code block at s * 8192, its chunk's scale block at (s / 2) * 1024, its
// token bytes at ks * 64 within each token row.
struct Pipe4Off {
  int w, s, t;
};
__device__ __forceinline__ Pipe4Off pipe4_offsets(int s, int nk) {
  const int seg = s / nk, ks = s - seg * nk;
  return {s * Pipe4::W_BYTES, (s >> 1) * Pipe4::SC_BYTES, ks * Pipe4::TROWB};
}

// Load q of a stage into ring buffer st: weight codes for q < WL, then token rows.
__device__ __forceinline__ void pipe4_issue_one(const Pipe4Rows& r, uint8_t* st, Pipe4Off o, int q) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = Pipe4;
  const int w = p4_wave();
  if (q < P::WL) {
    const uint32_t ow = static_cast<uint32_t>(((q * P::NWAVE + w) * 64 + (threadIdx.x & 63)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.wrs, (lds_void_t*)(st + (q * P::NWAVE + w) * 1024), 16, ow, o.w, 0, 0);
  } else {
    const int qq = q - P::WL;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.trs, (lds_void_t*)(st + P::T_OFF + (qq * P::NWAVE + w) * 1024), 16,
                                             r.ot[qq], o.t, 0, 0);
  }
#endif
}

// Scales of the chunk whose first stage is s (o = pipe4_offsets(s, ...)), by
// wave 0 into chunk slot (s / 2) % SC_SLOTS; issued before that stage's loads.
__device__ __forceinline__ void pipe4_issue_scales(const Pipe4Rows& r, uint8_t* lds, int s, Pipe4Off o) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = Pipe4;
  if (p4_wave() == 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.srs, (lds_void_t*)(lds + P::SC_OFF + ((s >> 1) % P::SC_SLOTS) * P::SC_BYTES),
                                             16, static_cast<uint32_t>((threadIdx.x & 63) * 16), o.s, 0, 0);
#endif
}

// s_waitcnt vmcnt + barrier, with wave 0 allowing W0 loads in flight and the
// other waves W (wave 0 has issued the chunks' scale loads besides).
template <int W0, int W>
__device__ __forceinline__ void pipe4_wait_barrier() {
  if (p4_wave() == 0)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(W0) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(W) : "memory");
}

// Token-scale table of the tile (as pipe8_issue_scale_table, at Pipe4's offsets).
__device__ __forceinline__ void pipe4_issue_scale_table(__amdgpu_buffer_rsrc_t srs, uint8_t* lds, int kc, int kc_pad) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = Pipe4;
  const int tid = threadIdx.x, w = p4_wave();
  const int* src = reinterpret_cast<const int*>(lds + P::SRC_OFF);
  for (int q = 0; q < kc_pad * P::BT / P::NT; ++q) {
    const int e = q * P::NT + tid, r = e / kc_pad, c = min(e - r * kc_pad, kc - 1);
    const uint32_t off = (static_cast<uint32_t>(src[r]) * kc + c) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void_t*)(lds + P::SA_OFF + (q * P::NT + w * 64) * 4), 4, off, 0,
                                             0, 0);
  }
#endif
}

template <int MS>
struct Pipe4Frags {
  i32x8 w[Pipe4::TW];      // E2M1: the low four dwords are read
  int s[Pipe4::TW];        // E8M0 scale byte of this lane's 32-value block
  i32x8 t[MS > 0 ? MS : 1];
};

// Fragments of stage g (ring buffer st); its scales are K blocks 2 (g & 1) and
// 2 (g & 1) + 1 of chunk slot (g / 2) % SC_SLOTS.
template <int MS>
__device__ __forceinline__ void pipe4_read(Pipe4Frags<MS>& f, const uint8_t* lds, int g) {
  using P = Pipe4;
  const uint8_t* st = lds + (g % P::NS) * P::STAGE;
  const uint8_t* sc = lds + P::SC_OFF + ((g >> 1) % P::SC_SLOTS) * P::SC_BYTES + (g & 1) * 2 * P::BW;
  const int l = threadIdx.x & 63, h = l >> 5, wt = p8_wt(), ww = p8_ww();
#pragma unroll
  for (int j = 0; j < P::TW; ++j) {
    const int row = ww * (P::BW / 2) + j * 32 + (l & 31);
    const u32x4 v = *reinterpret_cast<const u32x4*>(st + row * P::WROWB + ((h ^ ((row >> 3) & 1)) << 4));
    f.w[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    f.s[j] = sc[h * P::BW + row];
  }
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int row = 32 * (2 * i + wt) + (l & 31), sw = (row >> 2) & 3;
    const uint8_t* tr = st + P::T_OFF + row * P::TROWB;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(tr + ((h ^ sw) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(tr + (((h + 2) ^ sw) << 4));
    f.t[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

__device__ __forceinline__ f32x16 mfma_f4f8(const i32x8& w, const i32x8& t, const f32x16& c, int ws) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, t, c, 4, 0, 0, ws, 0, 127);
}

// Accumulator tile m = (j, i) moved to the next chunk's frame (factor of token sub-tile i).
template <int MS>
__device__ __forceinline__ void pipe4_rescale(f32x16 (&acc)[Pipe4::TW][Pipe4::TT], const float (&r)[Pipe4::TT],
                                              int m) {
  constexpr int D = MS > 0 ? MS : 1;
  const int j = m / D, i = m % D;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[j][i][v] *= r[i];
}

// One half of a stage's MFMAs, as pipe8_half: HALF 0 takes tiles [0, M/2),
// HALF 1 tiles [M/2, M) with the loads of stage `ls` (into ring buffer st)
// spread among them when ISSUE, preceded by its chunk's scale load when
// SCALES; SECOND (a chunk's second stage) moves tile m - 2 to the next frame
// right after MFMA m, a chunk's first stage moves tiles M - 2, M - 1 before
// MFMAs 0 and 1.
template <int MS, int LT, bool SECOND, int HALF, bool ISSUE, bool SCALES>
__device__ __forceinline__ void pipe4_half(const Pipe4Frags<MS>& f, f32x16 (&acc)[Pipe4::TW][Pipe4::TT],
                                           const float (&r)[Pipe4::TT], const Pipe4Rows& rows, uint8_t* lds, int ls,
                                           Pipe4Off lo) {
  using P = Pipe4;
  constexpr int M = P::TW * MS, D = MS > 0 ? MS : 1, H = M / 2;
  constexpr int M0 = HALF ? H : 0, N = HALF ? M - H : H;
  constexpr int L = ISSUE ? P::WL + LT : 0;
  uint8_t* st = lds + (ls % P::NS) * P::STAGE;
  if (SCALES) {
    pipe4_issue_scales(rows, lds, ls, lo);
    sched_fence();
  }
#pragma unroll
  for (int n = 0; n < (N > L ? N : L); ++n) {
#pragma unroll
    for (int q = 0; q < L; ++q)
      if ((N == 0 && q == n) || (N > 0 && q * N / (L > 0 ? L : 1) == n)) {
        pipe4_issue_one(rows, st, lo, q);
        sched_fence();
      }
    if (n < N) {
      const int m = M0 + n;
      if (!SECOND && m < 2) pipe4_rescale<MS>(acc, r, M - 2 + m);
      acc[m / D][m % D] = mfma_f4f8(f.w[m / D], f.t[m % D], acc[m / D][m % D], f.s[m / D]);
      if (SECOND && m >= 2) pipe4_rescale<MS>(acc, r, m - 2);
      sched_fence();
    }
  }
  sched_fence();
}

// Token scale of this lane's row of each live sub-tile i for chunk c.
template <int MS>
__device__ __forceinline__ void pipe4_token_scales(float (&sa)[Pipe4::TT], const uint8_t* lds, int kc_pad, int c) {
  const float* sat = reinterpret_cast<const float*>(lds + Pipe4::SA_OFF);
  const int l = threadIdx.x & 63, wt = p8_wt();
#pragma unroll
  for (int i = 0; i < MS; ++i) sa[i] = sat[(32 * (2 * i + wt) + (l & 31)) * kc_pad + c];
}

// Frame change into chunk c + 1: sa holds the token scales of chunk c + 1
// (of chunk c when c is the block's last, next = false).
template <int MS>
__device__ __forceinline__ void pipe4_frame_update(float (&fac)[Pipe4::TT], float (&r)[Pipe4::TT],
                                                   const float (&sa)[Pipe4::TT], bool next) {
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const float fn = fmaxf(sa[i], kMinFactor);
    r[i] = next ? fac[i] * __builtin_amdgcn_rcpf(fn) : 1.0f;
    fac[i] = fn;
  }
}

// One stage of the stream (global index g, local index kt of output-column
// block seg): the first half of its MFMAs; then, unless it is the stream's last
// stage (W < 0), wait until stage g+1 and its scales have landed (wave 0 may
// keep W0 loads in flight, the others W) + barrier, and read stage g+1's
// fragments; the second half of the MFMAs, with the loads of stage g+NS-1 spread
// among them when ISSUE (into the buffer of stage g-1, which every wave has
// finished with), and before them that stage's chunk scales when it starts a
// chunk (g even: the first stage of a pair; the scales of chunk c + 3 go into
// the slot chunk c - 1 held, read for the last time before the barrier of
// stage 2c - 1). A chunk's first stage also reads the next chunk's token
// scales before its MFMAs and forms the frame change after them.
template <int MS, int LT, bool SECOND, int W0, int W, bool ISSUE>
__device__ __forceinline__ void pipe4_stage(const Pipe4Rows& rows, uint8_t* lds, int kc_pad, int kt, int g, int nk,
                                            const Pipe4Frags<MS>& fa, Pipe4Frags<MS>& fb,
                                            f32x16 (&acc)[Pipe4::TW][Pipe4::TT], float (&fac)[Pipe4::TT],
                                            float (&r)[Pipe4::TT]) {
  using P = Pipe4;
  const bool next = (kt >> 1) + 1 < (nk >> 1);
  float sa[P::TT];
  if (!SECOND) pipe4_token_scales<MS>(sa, lds, kc_pad, next ? (kt >> 1) + 1 : kt >> 1);
  sched_fence();
  pipe4_half<MS, LT, SECOND, 0, false, false>(fa, acc, r, rows, lds, 0, Pipe4Off{0, 0, 0});
  if (W >= 0) {
    pipe4_wait_barrier<(W0 >= 0 ? W0 : 0), (W >= 0 ? W : 0)>();
    pipe4_read<MS>(fb, lds, g + 1);
    sched_fence();
  }
  const int ls = ISSUE ? g + P::NS - 1 : 0;
  const Pipe4Off lo = ISSUE ? pipe4_offsets(ls, nk) : Pipe4Off{0, 0, 0};
  // stage g + NS - 1 starts a chunk when g is even: the first stage of a pair
  static_assert(P::NS % 2 == 1, "an odd ring: the issued stage starts a chunk in the pair's first stage");
  pipe4_half<MS, LT, SECOND, 1, ISSUE, ISSUE && !SECOND>(fa, acc, r, rows, lds, ls, lo);
  if (!SECOND) pipe4_frame_update<MS>(fac, r, sa, next);
}

// End of output-column block seg: acc times the last chunk's token scale for
// the epilogue, then acc restarts from zero in the frame of the next block's
// first chunk.
template <int MS, class EPI>
__device__ __forceinline__ void pipe4_finish(f32x16 (&acc)[Pipe4::TW][Pipe4::TT], float (&fac)[Pipe4::TT], EPI& epi,
                                             int seg, int nseg, const uint8_t* lds, int kc_pad) {
#pragma unroll
  for (int j = 0; j < Pipe4::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] *= fac[i];
  epi(seg, acc);
#pragma unroll
  for (int j = 0; j < Pipe4::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  if (seg + 1 < nseg) {
    float sa[Pipe4::TT];
    pipe4_token_scales<MS>(sa, lds, kc_pad, 0);
#pragma unroll
    for (int i = 0; i < MS; ++i) fac[i] = fmaxf(sa[i], kMinFactor);
  }
}

// Two consecutive stages g, g+1 (a chunk) of the stream, then the end of the
// output-column block if the chunk was its last. A0/B0 and A1/B1: loads wave 0
// and the other waves may keep in flight at the two barriers (B1 < 0: the
// stream's last stage, no barrier); I0/I1: stages g+NS-1 and g+NS exist and are
// loaded.
template <int MS, int LT, int A0, int B0, bool I0, int A1, int B1, bool I1, class EPI>
__device__ __forceinline__ void pipe4_pair(const Pipe4Rows& rows, uint8_t* lds, int kc_pad, int& kt, int g, int nk,
                                           int& seg, int nseg, Pipe4Frags<MS>& f0, Pipe4Frags<MS>& f1,
                                           f32x16 (&acc)[Pipe4::TW][Pipe4::TT], float (&fac)[Pipe4::TT],
                                           float (&r)[Pipe4::TT], EPI& epi) {
  pipe4_stage<MS, LT, false, A0, B0, I0>(rows, lds, kc_pad, kt, g, nk, f0, f1, acc, fac, r);
  pipe4_stage<MS, LT, true, A1, B1, I1>(rows, lds, kc_pad, kt + 1, g + 1, nk, f1, f0, acc, fac, r);
  kt += 2;
  if (kt == nk) {
    pipe4_finish<MS>(acc, fac, epi, seg, nseg, lds, kc_pad);
    ++seg;
    kt = 0;
  }
}

// The K loops of nseg output-column blocks of one unit as one stream of
// total = nseg * nk stages (as pipe8_stream, with a seven-stage ring); rows.wrs
// and rows.srs start at the unit's first column block. K % 128 == 0, K / 128 <= MAX_CHUNKS,
// nseg <= MAX_SEG. Before the call the unit's source rows are in LDS and
// visible to every wave. At the barrier of stage g every issued stage after
// g+1 (at most four: g+2 .. g+5) may still be in flight, and for wave 0 the
// scale loads of the chunks among them (two: the chunks start on even stages);
// loads complete in issue order, so a stage's scales, issued just before it,
// have landed with it. The last six stages are peeled so every wait is a
// constant.
template <int MS, int LT, class EPI>
__device__ __forceinline__ void pipe4_stream(const Pipe4Rows& rows, __amdgpu_buffer_rsrc_t tsrs, int K, int nseg,
                                             uint8_t* lds, EPI& epi) {
  using P = Pipe4;
  static_assert(P::NS == 7, "schedule written for a ring of seven stages");
  static_assert(LT >= 1 && LT <= P::TL && LT >= MS, "token load groups must cover the live sub-tiles");
  constexpr int L = P::WL + LT;                        // stage loads per thread (wave 0: + 1 per chunk)
  const int nk = K / P::BK, kc = K / 128, kc_pad = (kc + 3) & ~3, total = nseg * nk;   // nk even, total >= 2
  pipe4_issue_scale_table(tsrs, lds, kc, kc_pad);
  for (int s = 0; s < P::NS - 1 && s < total; ++s) {
    const Pipe4Off o = pipe4_offsets(s, nk);
    if ((s & 1) == 0) pipe4_issue_scales(rows, lds, s, o);
#pragma unroll
    for (int q = 0; q < L; ++q) pipe4_issue_one(rows, lds + s * P::STAGE, o, q);
  }
  // the token-scale table, stage 0 and its scales have landed; stages 1 .. min(5, total - 1) (wave 0: and the
  // scales of stages 2 and 4) may be in flight
  if (total >= 6) pipe4_wait_barrier<5 * L + 2, 5 * L>();
  else if (total == 4) pipe4_wait_barrier<3 * L + 1, 3 * L>();
  else pipe4_wait_barrier<L, L>();                     // total == 2
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0xc07f);                  // no scalar load pending: LDS waits stay partial
#endif
  f32x16 acc[P::TW][P::TT];
  float fac[P::TT], r[P::TT];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    r[i] = 1.0f;
#pragma unroll
    for (int j = 0; j < P::TW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  }
  {
    float sa[P::TT];
    pipe4_token_scales<MS>(sa, lds, kc_pad, 0);
#pragma unroll
    for (int i = 0; i < MS; ++i) fac[i] = fmaxf(sa[i], kMinFactor);
  }
  Pipe4Frags<MS> f0, f1;
  pipe4_read<MS>(f0, lds, 0);
  int kt = 0, seg = 0, g = 0;
  // steady state: each stage of the pair loads the stage six ahead; in flight at the first barrier g+2..g+5,
  // at the second g+3..g+6 (two chunk starts either way)
  for (; g + 8 <= total; g += 2)
    pipe4_pair<MS, LT, 4 * L + 2, 4 * L, true, 4 * L + 2, 4 * L, true>(rows, lds, kc_pad, kt, g, nk, seg, nseg, f0, f1,
                                                                       acc, fac, r, epi);
  if (total - g == 6) {                               // nothing left to issue: g+2..g+5, then g+3..g+5
    pipe4_pair<MS, LT, 4 * L + 2, 4 * L, false, 3 * L + 1, 3 * L, false>(rows, lds, kc_pad, kt, g, nk, seg, nseg, f0,
                                                                         f1, acc, fac, r, epi);
    g += 2;
  }
  if (total - g == 4) {
    pipe4_pair<MS, LT, 2 * L + 1, 2 * L, false, L, L, false>(rows, lds, kc_pad, kt, g, nk, seg, nseg, f0, f1, acc,
                                                             fac, r, epi);
    g += 2;
  }
  pipe4_pair<MS, LT, 0, 0, false, -1, -1, false>(rows, lds, kc_pad, kt, g, nk, seg, nseg, f0, f1, acc, fac, r,
                                                 epi);
  // every wave has read the ring before the next unit's loads overwrite it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe
