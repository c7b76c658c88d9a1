// Measured peaks of the GPU the library runs on, for the roofline figures:
// an MFMA loop (bf16 32x32x16 and E4M3 32x32x64 with unit block scales, eight
// independent accumulators per wave so the matrix pipe never waits on a
// result), a 16-byte-per-lane stream copy and a read-only stream. Neither is on the layer's path.
#include "common.h"
#include "launch.h"

namespace moe {

template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, const int* __restrict__ seed, float* __restrict__ out) {
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
  const int s = seed[threadIdx.x & 63];
  if (FP8) {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = s * (i + 1) & 0x3B3B3B3B;       // small finite E4M3 codes
      b[i] = s * (i + 3) & 0x3A3A3A3A;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, 127, 0, 127);
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<__bf16>(static_cast<float>((s + i) & 7) * 0.125f);
      b[i] = static_cast<__bf16>(static_cast<float>((s + 2 * i) & 7) * 0.125f);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = mfma_32x32x16_bf16(a, b, acc[i]);
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) t += acc[i][v];
  out[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = t;   // keeps the loop
}

__global__ __launch_bounds__(256) void stream_copy_kernel(long long n16, const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst) {
  for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<long long>(gridDim.x) * 256)
    dst[i] = src[i];
}

// Read-only stream: every lane folds its 16-byte loads into one word (written, so the loads stay).
__global__ __launch_bounds__(256) void stream_read_kernel(long long n16, const uint4* __restrict__ src,
                                                          uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<long long>(gridDim.x) * 256) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

int probe_mfma_blocks() { return device_cu_count() * 2; }
int probe_read_blocks() { return device_cu_count() * 8; }

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(probe_read_blocks())), dim3(256), 0, st,
                     static_cast<long long>(bytes / 16), static_cast<const uint4*>(src), out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(bool fp8, int iters, const int* seed, float* out, hipStream_t st) {
  const dim3 g(static_cast<unsigned>(probe_mfma_blocks()));
  if (fp8) hipLaunchKernelGGL(mfma_loop_kernel<true>, g, dim3(256), 0, st, iters, seed, out);
  else hipLaunchKernelGGL(mfma_loop_kernel<false>, g, dim3(256), 0, st, iters, seed, out);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const long long n16 = static_cast<long long>(bytes / 16);
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(device_cu_count() * 8)), dim3(256), 0, st, n16,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst));
  return hipGetLastError();
}

}  // namespace moe
