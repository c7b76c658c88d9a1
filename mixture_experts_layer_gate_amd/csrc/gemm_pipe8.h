// Pipelined E4M3 MFMA main loop with the scales applied per 128-wide K
// chunk, for the fp8 expert GEMMs ("DeepSeek_V3_Report: Annotation",
// sections "Fine-Grained Quantization" and "Increasing Accumulation
// Precision").
//
// Operands are E4M3 codes: weights with one fp32 scale per 128x128 block,
// tokens with one fp32 scale per 1x128 tile, so output element (w, n) needs
// y = sum over chunks c of f_c * raw_c with f_c = s_token[n, c] *
// s_weight[block(w), c] and raw_c the chunk's code dot product. gfx950's
// block-scaled MFMA takes power-of-two scales only, so the fp32 factors are
// applied on the VALU; its MFMA accumulates fp8 products in fp32, so no
// separate low-precision partial sum needs promoting. The accumulator is kept
// in the frame of the current chunk, acc = (sum over c' <= c of f_c' *
// raw_c') / f_c: the two v_mfma_scale_f32_32x32x64_f8f6f4 of chunk c add raw_c
// to it directly, and between chunks it is multiplied by f_c / f_{c+1} (one
// VALU multiply per element per chunk); the epilogue multiplies by the last
// chunk's factor. Factors below 1e-20 are raised to 1e-20 so the frame never
// overflows; that changes no output by more than about 3e-13.
//
// Tile: BW = 256 weight rows x BT = 128 token rows, four waves (one per
// SIMD) in a 2 x 2 grid of 128 x 64: TW = 4 weight sub-tiles x up to 2 token
// sub-tiles of 32x32, 128 accumulator VGPRs per wave.
// Weight and token rows stream into LDS with buffer_load ... lds through a
// ring of four stages of 64 K-bytes (one MFMA K-step), rows of 64 bytes
// XOR-swizzled as in the bf16 loop. The tile's token scales (128 rows x all
// chunks) and weight scales are loaded into LDS tables once per tile: loaded
// per stage, the 4-byte scales of 128 scattered rows cost more L2 requests
// than the stage's 24 KB of operands.
//
// Iteration kt (stage kt, chunk kt / 2): the first half of stage kt's MFMAs;
// wait until stage kt+1 has landed + barrier; read stage kt+1's fragments;
// the second half of the MFMAs with the loads of stage kt+3 spread among them. A chunk's first stage prepares the next
// chunk's factors behind its MFMAs; its second stage moves each accumulator
// tile to the next frame two MFMAs after the tile's last MFMA of the chunk
// (the last two tiles at the start of the next stage), so the multiplies run
// beside the MFMAs. A unit streams up to
// MAX_SEG blocks of output columns that share its token rows as one sequence
// of stages, so the ring's fill and drain and the unit's setup are paid once
// per unit.
#pragma once

#include "common.h"
#include "gemm_pipe.h"

namespace moe {

struct Pipe8 {
  static constexpr int BW = 256, BT = 128, BK = 64, NS = 4, NT = 256, NWAVE = NT / 64;
  static constexpr int TW = 4, TT = 2;                    // 32x32 sub-tiles per wave
  static constexpr int ROWB = BK;                          // bytes per row per stage
  static constexpr int W_BYTES = BW * ROWB, T_BYTES = BT * ROWB;
  static constexpr int STAGE = W_BYTES + T_BYTES;
  static constexpr int WL = W_BYTES / 16 / NT, TL = T_BYTES / 16 / NT;
  static constexpr int LPS = WL + TL;                      // loads per thread per stage (all token groups)
  static constexpr int RING = NS * STAGE;
  static constexpr int MAX_CHUNKS = 80;                    // K <= 10240
  static constexpr int MAX_SEG = 4;                        // output-column blocks streamed per unit
  static constexpr int SW_OFF = RING;                      // weight scales [MAX_SEG][2][MAX_CHUNKS]
  static constexpr int SA_OFF = SW_OFF + MAX_SEG * 2 * MAX_CHUNKS * 4;   // token scales [BT][kc_pad]
  static constexpr int SRC_OFF = SA_OFF + BT * MAX_CHUNKS * 4;           // source row of each tile row [BT]
  static constexpr int AMAX_OFF = SRC_OFF + BT * 4;                      // epilogue exchange [2][BT]
  static constexpr int LDS_BYTES = AMAX_OFF + 2 * BT * 4;
  static_assert(WL * NT * 16 == W_BYTES && TL * NT * 16 == T_BYTES, "stage must split evenly over the threads");
  static_assert(LPS * 3 <= 63, "vmcnt range");
  static_assert((BT * 4) % NT == 0, "four chunks of the scale table split evenly over the threads");
};

// Wave coordinates: token half wt (rows 32 * (2i + wt) + lane % 32), weight
// half ww (tile rows 128 ww .. 128 ww + 127).
__device__ __forceinline__ int p8_wt() { return (threadIdx.x >> 6) & 1; }
__device__ __forceinline__ int p8_ww() { return threadIdx.x >> 7; }

// Tile row and logical 16-byte chunk of load q of this thread (16 rows of 64
// bytes per wave instruction).
__device__ __forceinline__ int pipe8_load_row(int q) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  return (q * Pipe8::NWAVE + w) * 16 + (l >> 2);
}
__device__ __forceinline__ int pipe8_load_chunk(int q) {
  const int l = threadIdx.x & 63;
  return (l & 3) ^ ((pipe8_load_row(q) >> 2) & 3);
}

// Operands: the unit's weight blocks (from its first column block on) and the
// token codes through buffer resources; token loads with 32-bit byte offsets
// (row * K + logical chunk * 16). Weight load q of a thread reads the 16 bytes
// at ((q * NWAVE + wave) * 64 + lane) * 16 of the stage's block, which is the
// stage's LDS image.
struct Pipe8Rows {
  __amdgpu_buffer_rsrc_t wrs, trs;
  uint32_t ot[Pipe8::TL];
};

// A stage of the stream: output-column block seg = s / nk, K bytes
// (s % nk) * 64 .. +63. The weights are in the tiled layout of
// moe_quantize_weights, whose stage blocks of 16 KB follow each other for
// consecutive K steps and column blocks: the stage's weights are the block at
// s * 16 KB from the unit's first.
struct Pipe8Off {
  int w, t;   // SGPR byte offsets of the stage's weight and token loads
};
__device__ __forceinline__ Pipe8Off pipe8_offsets(int s, int nk) {
  const int seg = s / nk, ks = s - seg * nk;
  return {s * Pipe8::W_BYTES, ks * Pipe8::BK};
}

// Load q of a stage into ring buffer st: weights for q < WL, then token rows.
__device__ __forceinline__ void pipe8_issue_one(const Pipe8Rows& r, uint8_t* st, Pipe8Off o, int q) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = Pipe8;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (q < P::WL) {
    const uint32_t ow = static_cast<uint32_t>(((q * P::NWAVE + w) * 64 + (threadIdx.x & 63)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.wrs, (lds_void_t*)(st + (q * P::NWAVE + w) * 1024), 16, ow, o.w, 0, 0);
  } else {
    const int qq = q - P::WL;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.trs, (lds_void_t*)(st + P::W_BYTES + (qq * P::NWAVE + w) * 1024), 16,
                                             r.ot[qq], o.t, 0, 0);
  }
#endif
}

// Token-scale table of the tile: entry (r, c) = scales[src[r] * kc + min(c, kc-1)]
// at LDS float r * kc_pad + c, kc_pad = kc rounded up to a multiple of 4 so each
// thread issues exactly kc_pad / 4 dword loads (a wave's load covers 64
// consecutive entries: one or a few rows, contiguous in memory). The loads
// count in vmcnt like the ring's and complete at the prologue's wait.
__device__ __forceinline__ void pipe8_issue_scale_table(__amdgpu_buffer_rsrc_t srs, uint8_t* lds, int kc, int kc_pad) {
#if defined(__HIP_DEVICE_COMPILE__)
  using P = Pipe8;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
struct Pipe8Frags {
  i32x8 w[Pipe8::TW];
  i32x8 t[MS > 0 ? MS : 1];
};

// Fragment of tile row `row` (its 64-byte stage row): lane half h holds K bytes
// 32h .. 32h+31, i.e. logical chunks 2h and 2h+1, stored at chunk ^ ((row >> 2) & 3).
__device__ __forceinline__ i32x8 pipe8_frag(const uint8_t* st, int row) {
  const int l = threadIdx.x & 63, sw = (row >> 2) & 3, c0 = 2 * (l >> 5);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(st + row * Pipe8::ROWB + ((c0 ^ sw) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(st + row * Pipe8::ROWB + (((c0 + 1) ^ sw) << 4));
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int MS>
__device__ __forceinline__ void pipe8_read(Pipe8Frags<MS>& f, const uint8_t* st) {
  const int l = threadIdx.x & 63, wt = p8_wt(), ww = p8_ww();
#pragma unroll
  for (int j = 0; j < Pipe8::TW; ++j) f.w[j] = pipe8_frag(st, ww * (Pipe8::BW / 2) + j * 32 + (l & 31));
#pragma unroll
  for (int i = 0; i < MS; ++i) f.t[i] = pipe8_frag(st + Pipe8::W_BYTES, 32 * (2 * i + wt) + (l & 31));
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

constexpr float kMinFactor = 1e-20f;

// Accumulator tile t = (j, i) = (t / MS, t % MS) moved to the next chunk's frame.
template <int MS>
__device__ __forceinline__ void pipe8_rescale(f32x16 (&acc)[Pipe8::TW][Pipe8::TT],
                                              const float (&r)[Pipe8::TW][Pipe8::TT], int t) {
  constexpr int D = MS > 0 ? MS : 1;
  const int j = t / D, i = t % D;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[j][i][v] *= r[j][i];
}

// One half of a stage's MFMAs (fragments f), tile m = (m / MS, m % MS) in
// order: HALF 0 takes tiles [0, M/2), HALF 1 tiles [M/2, M) with the loads of
// stage `ls` spread among them (load q before the MFMA at q * H / L) when
// ISSUE. SECOND (a chunk's second stage): tile m - 2 moves to the next frame
// right after MFMA m; otherwise (a chunk's first stage) tiles M - 2 and M - 1,
// whose last MFMAs closed the previous stage, move before MFMAs 0 and 1.
template <int MS, int LT, bool SECOND, int HALF, bool ISSUE>
__device__ __forceinline__ void pipe8_half(const Pipe8Frags<MS>& f, f32x16 (&acc)[Pipe8::TW][Pipe8::TT],
                                           const float (&r)[Pipe8::TW][Pipe8::TT], const Pipe8Rows& rows,
                                           uint8_t* lds, int ls, Pipe8Off lo) {
  using P = Pipe8;
  constexpr int M = P::TW * MS, D = MS > 0 ? MS : 1, H = M / 2;
  constexpr int M0 = HALF ? H : 0, N = HALF ? M - H : H;      // this half's first MFMA, count
  constexpr int L = ISSUE ? P::WL + LT : 0;                   // weight loads, then LT token load groups
  uint8_t* st = lds + (ls & 3) * P::STAGE;
#pragma unroll
  for (int n = 0; n < (N > L ? N : L); ++n) {
#pragma unroll
    for (int q = 0; q < L; ++q)
      if ((N == 0 && q == n) || (N > 0 && q * N / (L > 0 ? L : 1) == n)) {
        pipe8_issue_one(rows, st, lo, q);
        sched_fence();
      }
    if (n < N) {
      const int m = M0 + n;
      if (!SECOND && m < 2) pipe8_rescale<MS>(acc, r, M - 2 + m);
      acc[m / D][m % D] = mfma_f8(f.w[m / D], f.t[m % D], acc[m / D][m % D]);
      if (SECOND && m >= 2) pipe8_rescale<MS>(acc, r, m - 2);
      sched_fence();
    }
  }
  sched_fence();
}

// Factors of chunk c of output-column block seg: token scale of this lane's
// row of sub-tile i times the weight-block scale of sub-tile j (gate/up
// tiles: block row 0 for the gate sub-tiles j < TW / 2, 1 for the up
// sub-tiles; down tiles: the 128-row block of this wave's rows).
template <int MS, bool GATE_UP>
__device__ __forceinline__ void pipe8_factors(float (&fac)[Pipe8::TW][Pipe8::TT], const uint8_t* lds, int kc_pad,
                                              int c, int seg) {
  const float* swt = reinterpret_cast<const float*>(lds + Pipe8::SW_OFF) + seg * 2 * Pipe8::MAX_CHUNKS;
  const float* sat = reinterpret_cast<const float*>(lds + Pipe8::SA_OFF);
  const int l = threadIdx.x & 63, wt = p8_wt();
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const float sa = sat[(32 * (2 * i + wt) + (l & 31)) * kc_pad + c];
#pragma unroll
    for (int j = 0; j < Pipe8::TW; ++j)
      fac[j][i] = fmaxf(sa * swt[(GATE_UP ? (j >= Pipe8::TW / 2 ? 1 : 0) : p8_ww()) * Pipe8::MAX_CHUNKS + c],
                        kMinFactor);
  }
}

// The scales behind the factors of one chunk, read from the LDS tables: the
// token scale of this lane's row of each sub-tile i, and the weight-block
// scale(s) (gate/up tiles: [0] gate block, [1] up block; down tiles: [0] the
// 128-row block of this wave's rows).
struct Pipe8Scales {
  float sa[Pipe8::TT];
  float sw[2];
};

template <int MS, bool GATE_UP>
__device__ __forceinline__ void pipe8_scale_loads(Pipe8Scales& sc, const uint8_t* lds, int kc_pad, int c, int seg) {
  const float* swt = reinterpret_cast<const float*>(lds + Pipe8::SW_OFF) + seg * 2 * Pipe8::MAX_CHUNKS;
  const float* sat = reinterpret_cast<const float*>(lds + Pipe8::SA_OFF);
  const int l = threadIdx.x & 63, wt = p8_wt();
#pragma unroll
  for (int i = 0; i < MS; ++i) sc.sa[i] = sat[(32 * (2 * i + wt) + (l & 31)) * kc_pad + c];
  sc.sw[0] = swt[(GATE_UP ? 0 : p8_ww()) * Pipe8::MAX_CHUNKS + c];
  sc.sw[1] = GATE_UP ? swt[Pipe8::MAX_CHUNKS + c] : sc.sw[0];
}

// Frame change into chunk c + 1 of the same block: sc holds the scales of
// chunk c + 1 (of chunk c when c is the block's last, next = false).
// r = f_c / f_{c+1} and fac becomes f_{c+1}; for the last chunk r = 1 and fac
// stays f_c for the epilogue.
template <int MS, bool GATE_UP>
__device__ __forceinline__ void pipe8_frame_update(float (&fac)[Pipe8::TW][Pipe8::TT],
                                                   float (&r)[Pipe8::TW][Pipe8::TT], const Pipe8Scales& sc,
                                                   bool next) {
#pragma unroll
  for (int j = 0; j < Pipe8::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const float fn = fmaxf(sc.sa[i] * sc.sw[GATE_UP && j >= Pipe8::TW / 2 ? 1 : 0], kMinFactor);
      r[j][i] = next ? fac[j][i] * __builtin_amdgcn_rcpf(fn) : 1.0f;
      fac[j][i] = fn;
    }
}

// One stage of the stream (global index g, local index kt within its
// output-column block seg): fa holds its fragments, fb receives stage g+1's.
// The first half of its MFMAs runs before the barrier, so the MFMA pipe still
// has queued work while the wave waits there; after the barrier it reads stage
// g+1's fragments and issues the second half with stage g+3's loads (into the
// buffer of stage g-1, which every wave has finished with once it has issued
// stage g's first MFMAs). WAIT: loads allowed in flight at the barrier (one
// stage's while stage g+2 exists, else 0), or -1 for the stream's last stage
// (no barrier, nothing to read); ISSUE: load stage g+3. A chunk's first stage
// also reads the next chunk's scales (before its MFMAs) and forms the frame
// change (after them), so the second stage's multiplies find r ready.
template <int MS, int LT, bool GATE_UP, bool SECOND, int WAIT, bool ISSUE>
__device__ __forceinline__ void pipe8_stage(const Pipe8Rows& rows, uint8_t* lds, int kc_pad, int kt, int g, int nk,
                                            int seg, const Pipe8Frags<MS>& fa, Pipe8Frags<MS>& fb,
                                            f32x16 (&acc)[Pipe8::TW][Pipe8::TT], float (&fac)[Pipe8::TW][Pipe8::TT],
                                            float (&r)[Pipe8::TW][Pipe8::TT]) {
  using P = Pipe8;
  const bool next = (kt >> 1) + 1 < (nk >> 1);
  Pipe8Scales sc;
  if (!SECOND) pipe8_scale_loads<MS, GATE_UP>(sc, lds, kc_pad, next ? (kt >> 1) + 1 : kt >> 1, seg);
  sched_fence();
  pipe8_half<MS, LT, SECOND, 0, false>(fa, acc, r, rows, lds, 0, Pipe8Off{0, 0});
  if (WAIT >= 0) {
    wait_vm_only_barrier<(WAIT >= 0 ? WAIT : 0)>();
    pipe8_read<MS>(fb, lds + ((g + 1) & 3) * P::STAGE);
    sched_fence();
  }
  const Pipe8Off lo = ISSUE ? pipe8_offsets(g + 3, nk) : Pipe8Off{0, 0};
  pipe8_half<MS, LT, SECOND, 1, ISSUE>(fa, acc, r, rows, lds, g + 3, lo);
  if (!SECOND) pipe8_frame_update<MS, GATE_UP>(fac, r, sc, next);
}

// End of output-column block seg: y = acc * (last chunk's factor) for the
// epilogue, then acc restarts from zero with the factors of the next block's
// first chunk.
template <int MS, bool GATE_UP, class EPI>
__device__ __forceinline__ void pipe8_finish(f32x16 (&acc)[Pipe8::TW][Pipe8::TT], float (&fac)[Pipe8::TW][Pipe8::TT],
                                             EPI& epi, int seg, int nseg, const uint8_t* lds, int kc_pad) {
#pragma unroll
  for (int j = 0; j < Pipe8::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] *= fac[j][i];
  epi(seg, acc);
#pragma unroll
  for (int j = 0; j < Pipe8::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  if (seg + 1 < nseg) pipe8_factors<MS, GATE_UP>(fac, lds, kc_pad, 0, seg + 1);
}

// The K loops of nseg output-column blocks of one unit as one stream of
// total = nseg * nk stages through the ring: the next block's stages are in
// flight while a block ends. For each block: acc = the block's outputs, then
// epi(seg, acc) (stores; may use AMAX_OFF with an LDS-only barrier).
// K % 128 == 0, K / 128 <= MAX_CHUNKS, nseg <= MAX_SEG. Before the call the
// unit's source rows and weight scales ([seg][2][chunk]) are in LDS and
// visible to every wave; the token-scale table is loaded here from srs
// (kc = K / 128 scales per source row). LT (>= MS of every wave) token load
// groups of 64 rows per stage.
template <int MS, int LT, bool GATE_UP, class EPI>
__device__ __forceinline__ void pipe8_stream(const Pipe8Rows& rows, __amdgpu_buffer_rsrc_t srs, int K, int nseg,
                                             uint8_t* lds, EPI& epi) {
  using P = Pipe8;
  static_assert(LT >= 1 && LT <= P::TL && LT >= MS, "token load groups must cover the live sub-tiles");
  constexpr int LPS = P::WL + LT;                      // loads per stage per thread
  const int nk = K / P::BK, kc = K / 128, kc_pad = (kc + 3) & ~3, total = nseg * nk;   // nk even, total >= 2
  pipe8_issue_scale_table(srs, lds, kc, kc_pad);
  for (int s = 0; s < 3 && s < total; ++s) {
    const Pipe8Off o = pipe8_offsets(s, nk);
#pragma unroll
    for (int q = 0; q < LPS; ++q) pipe8_issue_one(rows, lds + s * P::STAGE, o, q);
  }
  if (total >= 3) wait_vm_only_barrier<2 * LPS>();     // scale table and stage 0 have landed
  else wait_vm_only_barrier<LPS>();                    // total == 2
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0xc07f);                  // no scalar load pending: LDS waits stay partial
#endif
  f32x16 acc[P::TW][P::TT];
  float fac[P::TW][P::TT], r[P::TW][P::TT];
#pragma unroll
  for (int j = 0; j < P::TW; ++j)
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      r[j][i] = 1.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
    }
  pipe8_factors<MS, GATE_UP>(fac, lds, kc_pad, 0, 0);
  Pipe8Frags<MS> f0, f1;
  pipe8_read<MS>(f0, lds);
  int kt = 0, seg = 0, g = 0;
  for (; g + 4 < total; g += 2) {                      // both stages refill the ring
    pipe8_stage<MS, LT, GATE_UP, false, LPS, true>(rows, lds, kc_pad, kt, g, nk, seg, f0, f1, acc, fac, r);
    pipe8_stage<MS, LT, GATE_UP, true, LPS, true>(rows, lds, kc_pad, kt + 1, g + 1, nk, seg, f1, f0, acc, fac,
                                                  r);
    kt += 2;
    if (kt == nk) {
      pipe8_finish<MS, GATE_UP>(acc, fac, epi, seg, nseg, lds, kc_pad);
      ++seg;
      kt = 0;
    }
  }
  if (g + 4 == total) {                                // stage total-1 is the last to load
    pipe8_stage<MS, LT, GATE_UP, false, LPS, true>(rows, lds, kc_pad, kt, g, nk, seg, f0, f1, acc, fac, r);
    pipe8_stage<MS, LT, GATE_UP, true, LPS, false>(rows, lds, kc_pad, kt + 1, g + 1, nk, seg, f1, f0, acc, fac,
                                                   r);
    kt += 2;
    if (kt == nk) {
      pipe8_finish<MS, GATE_UP>(acc, fac, epi, seg, nseg, lds, kc_pad);
      ++seg;
      kt = 0;
    }
  }
  // the stream's last pair: stage total-1 reads nothing
  pipe8_stage<MS, LT, GATE_UP, false, 0, false>(rows, lds, kc_pad, kt, total - 2, nk, seg, f0, f1, acc, fac, r);
  pipe8_stage<MS, LT, GATE_UP, true, -1, false>(rows, lds, kc_pad, kt + 1, total - 1, nk, seg, f1, f0, acc, fac,
                                                r);
  pipe8_finish<MS, GATE_UP>(acc, fac, epi, seg, nseg, lds, kc_pad);
  // every wave has read the ring before the next unit's loads overwrite it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe
