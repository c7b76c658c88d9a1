// 128x128 block quantisation of bf16 expert weights to E4M3 with one fp32
// scale per block ("DeepSeek_V3_Report: Annotation", section "Fine-Grained
// Quantization"; scale from the block's max-abs, section "Online Quantization").
#include "common.h"
#include "launch.h"

namespace moe {

// One block of 256 threads per 128x128 tile; thread t covers row t/2,
// columns 64*(t%2) .. +63.
__global__ __launch_bounds__(256) void quantize_blocks_kernel(int rows, int cols, const uint16_t* __restrict__ w,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float wmax[4];
  const int bc = cols / 128, br = rows / 128;
  const long long blk = blockIdx.x;
  const long long mat = blk / (static_cast<long long>(br) * bc);
  const int rem = static_cast<int>(blk % (static_cast<long long>(br) * bc));
  const int bi = rem / bc, bj = rem % bc;
  const int r = bi * 128 + (threadIdx.x >> 1);
  const int c0 = bj * 128 + (threadIdx.x & 1) * 64;
  const size_t base = (static_cast<size_t>(mat) * rows + r) * cols + c0;
  float x[64];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint4 p = *reinterpret_cast<const uint4*>(w + base + 8 * v);
    const uint32_t ww[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * v + 2 * i] = __uint_as_float(ww[i] << 16);
      x[8 * v + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, __builtin_fabsf(x[i]));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* xi = x + 16 * v + 4 * i;
      o[i] = f32x4_to_e4m3(xi[0] * inv, xi[1] * inv, xi[2] * inv, xi[3] * inv);
    }
    *reinterpret_cast<uint4*>(q + base + 16 * v) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (threadIdx.x == 0)
    scale[(static_cast<size_t>(mat) * br + bi) * bc + bj] = amax > 0.0f ? amax / kE4M3Max : 1.0f;
}

hipError_t launch_quantize_weights(int n_mats, int rows, int cols, const void* w, void* codes, float* scale,
                                   hipStream_t st) {
  const long long blocks = static_cast<long long>(n_mats) * (rows / 128) * (cols / 128);
  hipLaunchKernelGGL(quantize_blocks_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, rows, cols,
                     static_cast<const uint16_t*>(w), static_cast<uint8_t*>(codes), scale);
  return hipGetLastError();
}

}  // namespace moe
