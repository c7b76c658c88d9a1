// Measured peaks of the GPU, for the benchmark's roofline figures: an MFMA
// loop (bf16 32x32x16 and E4M3 32x32x64 with unit block scales, eight
// independent accumulators per wave so the matrix pipe never waits on a
// result), a 16-byte-per-lane stream copy and a read-only stream.
//
// Measurement tooling, not part of the layer: built into its own library
// (libmoe_probe.so) with the plain C entry points at the end of this file,
// which the benchmark loads; libmoe.so neither contains nor calls them.
#include "common.h"

namespace moe_probe {

using namespace moe;

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

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

}  // namespace moe_probe

// C entry points. Each returns 0 on success, -1 on a bad argument, or the
// hipError_t of the launch. Buffers are device pointers; stream is a
// hipStream_t (NULL: the default stream).
extern "C" {

// Workgroups of probe_mfma (4 waves each) and of probe_read (256 threads each).
int probe_mfma_blocks(void) { return moe_probe::cu_count() * 2; }
int probe_read_blocks(void) { return moe_probe::cu_count() * 8; }

// iters x 8 independent MFMAs per wave on register operands: fp8 = 0 issues bf16
// 32x32x16 (32768 FLOP each), fp8 = 1 E4M3 32x32x64 (131072 FLOP each). seed: 64
// int32 operand bits; out: probe_mfma_blocks() * 256 floats, written.
int probe_mfma(int fp8, int iters, const int* seed, float* out, void* stream) {
  if (iters <= 0 || !seed || !out) return -1;
  const dim3 g(static_cast<unsigned>(probe_mfma_blocks()));
  auto st = static_cast<hipStream_t>(stream);
  if (fp8) hipLaunchKernelGGL(moe_probe::mfma_loop_kernel<true>, g, dim3(256), 0, st, iters, seed, out);
  else hipLaunchKernelGGL(moe_probe::mfma_loop_kernel<false>, g, dim3(256), 0, st, iters, seed, out);
  return static_cast<int>(hipGetLastError());
}

// dst = src over bytes (a multiple of 16, 16 bytes per lane).
int probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || src == dst || bytes % 16) return -1;
  hipLaunchKernelGGL(moe_probe::stream_copy_kernel, dim3(static_cast<unsigned>(moe_probe::cu_count() * 8)), dim3(256),
                     0, static_cast<hipStream_t>(stream), static_cast<long long>(bytes / 16),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst));
  return static_cast<int>(hipGetLastError());
}

// Reads bytes (a multiple of 16) of src; out: probe_read_blocks() * 256 uint32, written.
int probe_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (!src || !out || bytes % 16) return -1;
  hipLaunchKernelGGL(moe_probe::stream_read_kernel, dim3(static_cast<unsigned>(probe_read_blocks())), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<long long>(bytes / 16),
                     static_cast<const uint4*>(src), out);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
