// Epilogues of the grouped E4M3-activation FFN kernels (fp8 and MXFP4
// weights): the SwiGLU with the 1x128 re-quantisation of H after gate/up, the
// bf16 store after down. Both main loops (gemm_pipe8.h, gemm_pipe4.h) use
// tiles of 256 weight rows x 128 token rows in the same wave layout, so the
// accumulator of weight sub-tile j x token sub-tile i holds the same output
// elements in both.
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

// gate/up epilogue of output-column tile nb0 + seg: SwiGLU in fp32 (this wave
// holds 64 of the tile's 128 H columns of each row: gate sub-tiles 0, 1 with
// up sub-tiles 2, 3), then the 1x128 re-quantisation of H over the tile's
// 128 columns (row amax exchanged through LDS).
template <int MS, int AMAX_OFF>
struct GateUpEpi8 {
  const Unit& un;
  int I, nb0;
  uint8_t* lds;
  uint8_t* __restrict__ Hq;
  float* __restrict__ Hs;
  // backward cache (or NULL): the SwiGLU inputs [G, U] as 1x128 E4M3 tiles, rows of 2I codes and 2I/128 scales
  uint8_t* __restrict__ GUq = nullptr;
  float* __restrict__ GUs = nullptr;
  __device__ __forceinline__ void operator()(int seg, f32x16 (&acc)[P8::TW][P8::TT]) {
    const int l = threadIdx.x & 63, ww = p8_ww(), nb = nb0 + seg;
    float* amax_x = reinterpret_cast<float*>(lds + AMAX_OFF);   // [2][BT]
    float hv[P8::TT][2][16];
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      float x = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          hv[i][j][v] = silu(acc[j][i][v]) * acc[j + 2][i][v];
          x = fmaxf(x, __builtin_fabsf(hv[i][j][v]));
        }
      x = fmaxf(x, __shfl_xor(x, 32, kWave));
      if (l < 32) amax_x[ww * P8::BT + p8_token_row(i)] = x;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int tr = p8_token_row(i);
      const float amax = fmaxf(amax_x[tr], amax_x[P8::BT + tr]);
      if (tr < un.rows) {
        const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
        uint8_t* hrow = Hq + static_cast<size_t>(un.m0 + tr) * I + nb * 128 + ww * 64 + 4 * (l >> 5);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint32_t*>(hrow + j * 32 + 8 * q) =
                f32x4_to_e4m3(hv[i][j][4 * q] * inv, hv[i][j][4 * q + 1] * inv, hv[i][j][4 * q + 2] * inv,
                              hv[i][j][4 * q + 3] * inv);
        if (ww == 0 && l < 32) Hs[static_cast<size_t>(un.m0 + tr) * (I / 128) + nb] = amax > 0.0f ? amax / kE4M3Max : 1.0f;
      }
    }
    if (GUq != nullptr) {                              // G (sub-tiles 0, 1), then U (2, 3): same tile exchange
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        lds_barrier();                                  // every wave has read the previous amax_x
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          float x = 0.0f;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) x = fmaxf(x, __builtin_fabsf(acc[j + 2 * part][i][v]));
          x = fmaxf(x, __shfl_xor(x, 32, kWave));
          if (l < 32) amax_x[ww * P8::BT + p8_token_row(i)] = x;
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          const int tr = p8_token_row(i);
          const float amax = fmaxf(amax_x[tr], amax_x[P8::BT + tr]);
          if (tr < un.rows) {
            const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
            uint8_t* grow = GUq + static_cast<size_t>(un.m0 + tr) * 2 * I + part * I + nb * 128 + ww * 64 + 4 * (l >> 5);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x16& a = acc[j + 2 * part][i];
                *reinterpret_cast<uint32_t*>(grow + j * 32 + 8 * q) =
                    f32x4_to_e4m3(a[4 * q] * inv, a[4 * q + 1] * inv, a[4 * q + 2] * inv, a[4 * q + 3] * inv);
              }
            if (ww == 0 && l < 32)
              GUs[static_cast<size_t>(un.m0 + tr) * (2 * I / 128) + part * (I / 128) + nb] =
                  amax > 0.0f ? amax / kE4M3Max : 1.0f;
          }
        }
      }
    }
    // amax_x is next written in the following tile's epilogue, after at least
    // one ring barrier that every wave reaches with these reads consumed
  }
};

// down epilogue of output-column tile nb0 + seg: bf16 rows of y.
template <int MS>
struct DownEpi8 {
  const Unit& un;
  int d, nb0;
  uint16_t* __restrict__ y;
  float* __restrict__ yf = nullptr;   // fp32 rows instead (then y is unused)
  __device__ __forceinline__ void operator()(int seg, f32x16 (&acc)[P8::TW][P8::TT]) {
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int tr = p8_token_row(i);
      if (tr < un.rows) {
        const size_t row0 = static_cast<size_t>(un.m0 + tr) * d + (nb0 + seg) * P8::BW;
#pragma unroll
        for (int j = 0; j < P8::TW; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if ((nb0 + seg) * P8::BW + p8_wcol(j, q) < d) {  // the 128-column last tile of d % 256 == 128
              if (yf != nullptr)
                *reinterpret_cast<f32x4*>(yf + row0 + p8_wcol(j, q)) =
                    f32x4{acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
              else
                *reinterpret_cast<u32x2*>(y + row0 + p8_wcol(j, q)) =
                    u32x2{pack_bf16x2(acc[j][i][4 * q], acc[j][i][4 * q + 1]),
                          pack_bf16x2(acc[j][i][4 * q + 2], acc[j][i][4 * q + 3])};
            }
      }
    }
  }
};

}  // namespace moe
