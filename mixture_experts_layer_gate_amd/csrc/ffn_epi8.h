// Epilogues of the grouped E4M3-activation FFN kernels (fp8 and MXFP4
// weights): the SwiGLU with the 1x128 re-quantisation of H after gate/up, the
// bf16 store after down. The four-wave main loops (gemm_pipe8.h,
// gemm_pipe4.h) use tiles of 256 weight rows x 128 token rows in the same
// wave layout (P8Layout); the eight-wave fp8 loop (gemm_f8w.h) tiles of 256 x
// 256 (F8WLayout). In both a wave holds 4 weight sub-tiles (128 tile rows:
// for gate/up 64 gate rows, then the matching 64 up rows) x 2 token
// sub-tiles, and the layout class names the output element of each
// accumulator.
#pragma once

#include "common.h"
#include "gemm_pipe8.h"
#include "sched.h"

namespace moe {

using P8 = Pipe8;
constexpr int kMaxSub8 = P8::BT / 32;   // 32-row sub-tiles per block

__device__ __forceinline__ int live_token_subtiles8(int nsub) {
  return clampi((nsub - p8_wt() + 1) / 2, 0, P8::TT);
}

// Wave layout of the four-wave loops (see F8WLayout in gemm_f8w.h for the eight-wave one).
struct P8Layout {
  static constexpr int BW = P8::BW, BT = P8::BT, TW = P8::TW, TT = P8::TT;
  __device__ static int lane() { return threadIdx.x & 63; }
  __device__ static int ww() { return p8_ww(); }
  __device__ static int token_row(int i) { return 32 * (2 * i + p8_wt()) + (threadIdx.x & 31); }
  __device__ static int wcol(int j, int q) {
    return p8_ww() * (P8::BW / 2) + j * 32 + 8 * q + 4 * ((threadIdx.x & 63) >> 5);
  }
};

// Output column (weight row within the tile) of accumulator element 4q of
// weight sub-tile j: four consecutive columns per lane.
__device__ __forceinline__ int p8_wcol(int j, int q) {
  const int l = threadIdx.x & 63;
  return p8_ww() * (P8::BW / 2) + j * 32 + 8 * q + 4 * (l >> 5);
}

// Tile row of token sub-tile i of this lane.
__device__ __forceinline__ int p8_token_row(int i) {
  const int l = threadIdx.x & 63;
  return 32 * (2 * i + p8_wt()) + (l & 31);
}

// Barrier for LDS data only: the ring's loads stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The epilogues store through buffer resources that span exactly the block's
// rows (un.m0 .. un.m0 + un.rows - 1): a lane whose token row lies past the
// block is dropped by the range check, so the stores need no per-lane branch
// (a divergent branch around them keeps every accumulator live in a second
// register set).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, size_t row0, size_t row_bytes,
                                                           int rows) {
  return pipe_rsrc(static_cast<const uint8_t*>(base) + row0 * row_bytes, static_cast<uint64_t>(rows) * row_bytes);
}

// gate/up epilogue of output-column tile nb0 + seg: SwiGLU in fp32 (this wave
// holds 64 of the tile's 128 H columns of each row: gate sub-tiles 0, 1 with
// up sub-tiles 2, 3), then the 1x128 re-quantisation of H over the tile's
// 128 columns (row amax exchanged through LDS). With the backward cache, G
// and U are quantised first, so H can replace G in the accumulators.
template <int MS, int AMAX_OFF, class LY = P8Layout>
struct GateUpEpi8 {
  const Unit& un;
  int I, nb0;
  uint8_t* lds;
  uint8_t* __restrict__ Hq;
  float* __restrict__ Hs;
  // backward cache (or NULL): the SwiGLU inputs [G, U] as 1x128 E4M3 tiles, rows of 2I codes and 2I/128 scales
  uint8_t* __restrict__ GUq = nullptr;
  float* __restrict__ GUs = nullptr;
  // Row amax over the tile's 128 columns of sub-tiles j0, j0 + 1 exchanged through LDS; returns after the
  // barrier that makes both wave halves' values visible.
  __device__ __forceinline__ void exchange_amax(const f32x16 (&acc)[LY::TW][LY::TT], int j0, float* amax_x) {
    const int ww = LY::ww();
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      float x = 0.0f;
#pragma unroll
      for (int j = j0; j < j0 + 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) x = fmaxf(x, __builtin_fabsf(acc[j][i][v]));
      x = fmaxf(x, __shfl_xor(x, 32, kWave));
      amax_x[ww * LY::BT + LY::token_row(i)] = x;      // lanes l and l + 32: the same row and value
    }
    lds_barrier();
  }
  // 1x128 E4M3 codes of sub-tiles j0, j0 + 1 into rows of `stride` bytes of q (from byte col0 of a row)
  // and their scale into rows of sstride floats of sc (from float scol).
  __device__ __forceinline__ void store_tiles(const f32x16 (&acc)[LY::TW][LY::TT], int j0, const float* amax_x,
                                              uint8_t* __restrict__ q, int stride, int col0,
                                              float* __restrict__ sc, int sstride, int scol) {
    const int l = LY::lane(), ww = LY::ww();
    const __amdgpu_buffer_rsrc_t qr = rows_rsrc(q, un.m0, stride, un.rows);
    const __amdgpu_buffer_rsrc_t sr = rows_rsrc(sc, un.m0, 4 * static_cast<size_t>(sstride), un.rows);
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int tr = LY::token_row(i);
      const float amax = fmaxf(amax_x[tr], amax_x[LY::BT + tr]);
      const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
      const int off = tr * stride + col0 + ww * 64 + 4 * (l >> 5);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x16& a = acc[j0 + j][i];
          __builtin_amdgcn_raw_buffer_store_b32(
              f32x4_to_e4m3(a[4 * qq] * inv, a[4 * qq + 1] * inv, a[4 * qq + 2] * inv, a[4 * qq + 3] * inv), qr,
              off + j * 32 + 8 * qq, 0, 0);
        }
      if (ww == 0)                                       // lanes l and l + 32 store the same value
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, amax > 0.0f ? amax / kE4M3Max : 1.0f),
                                              sr, (tr * sstride + scol) * 4, 0, 0);
    }
  }
  __device__ __forceinline__ void operator()(int seg, f32x16 (&acc)[LY::TW][LY::TT]) {
    const int nb = nb0 + seg;
    float* amax_x = reinterpret_cast<float*>(lds + AMAX_OFF);   // [2][BT]
    if (GUq != nullptr) {                              // G (sub-tiles 0, 1), then U (2, 3)
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        if (part) lds_barrier();                        // every wave has read the previous amax_x
        exchange_amax(acc, 2 * part, amax_x);
        store_tiles(acc, 2 * part, amax_x, GUq, 2 * I, part * I + nb * 128, GUs, 2 * I / 128, part * (I / 128) + nb);
      }
      lds_barrier();
    }
    // H = SiLU(G) * U in place of G
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][i][v] = silu(acc[j][i][v]) * acc[j + 2][i][v];
    exchange_amax(acc, 0, amax_x);
    store_tiles(acc, 0, amax_x, Hq, I, nb * 128, Hs, I / 128, nb);
    // amax_x is next written in the following tile's epilogue, after at least
    // one ring barrier that every wave reaches with these reads consumed
  }
};

// down epilogue of output-column tile nb0 + seg: bf16 rows of y.
template <int MS, class LY = P8Layout, bool CHECK_COLS = true>
struct DownEpi8 {
  const Unit& un;
  int d, nb0;
  uint16_t* __restrict__ y;
  float* __restrict__ yf = nullptr;   // fp32 rows instead (then y is unused)
  template <bool F32>
  __device__ __forceinline__ void store(const f32x16 (&acc)[LY::TW][LY::TT], int col0) {
    constexpr int esz = F32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(F32 ? static_cast<void*>(yf) : static_cast<void*>(y), un.m0,
                                               static_cast<size_t>(d) * esz, un.rows);
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int off = (LY::token_row(i) * d + col0 + LY::wcol(0, 0)) * esz;
#pragma unroll
      for (int j = 0; j < LY::TW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (!CHECK_COLS || col0 + LY::wcol(j, q) < d) {   // the 128-column last tile of d % 256 == 128
            const f32x16& a = acc[j][i];
            if (F32)   // (the vector elements copied by value: a bit cast of an element lvalue reads element 0)
              __builtin_amdgcn_raw_buffer_store_b128(
                  u32x4{__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]), __float_as_uint(a[4 * q + 2]),
                        __float_as_uint(a[4 * q + 3])},
                  r, off + (j * 32 + 8 * q) * esz, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b64(
                  u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])}, r,
                  off + (j * 32 + 8 * q) * esz, 0, 0);
          }
    }
  }
  __device__ __forceinline__ void operator()(int seg, f32x16 (&acc)[LY::TW][LY::TT]) {
    const int col0 = (nb0 + seg) * LY::BW;
    if (yf != nullptr) store<true>(acc, col0);
    else store<false>(acc, col0);
  }
};

}  // namespace moe
