// moe_combine: eq. (12) of "DeepSeek_V3_Report: Annotation" -- residual plus
// the shared experts plus the gate-weighted routed experts, gathered per token
// (no atomics, so the result is deterministic), fp32 accumulation and one
// rounding. moe_bias_update: the step-end +-gamma rule of the same section.
#include "common.h"
#include "launch.h"

namespace moe {

__device__ __forceinline__ void ld8(const void* p, moe_dtype dt, size_t off, float (&x)[8]) {
  if (dt == MOE_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

constexpr int kMaxK = 16;

// bf16 rows of 8 channels: all loads of a row piece are issued before the first is used.
__device__ __forceinline__ uint4 ld_bf16x8(const void* p, size_t off) {
  return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
}
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// One block per token (grid-stride), d / 8 threads (at most 1024): each thread handles 8 consecutive
// channels, so at d <= 8192 a token takes one pass with all of its row loads in flight.
// KT > 0: bf16 rows and K = KT known at compile time, so the residual, the
// shared rows and the K routed rows of a piece are loaded together (K + 2
// loads in flight per lane instead of one) and then added in the same order
// as the general form: residual, shared experts, routed k = 0 .. K - 1.
template <int KT>
__global__ __launch_bounds__(1024) void combine_kernel(Shape s, moe_dtype io, const void* __restrict__ u,
                                                      const void* __restrict__ y, const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate,
                                                      const void* __restrict__ ysh, void* __restrict__ out) {
  __shared__ int rows[kMaxK];
  __shared__ float gts[kMaxK];
  const int d = s.d, K = KT > 0 ? KT : s.K;
  const long long n_rows = static_cast<long long>(s.T) * K;
  for (int t = blockIdx.x; t < s.T; t += gridDim.x) {
    if (threadIdx.x < K) {
      const int r = row_of[static_cast<size_t>(t) * K + threadIdx.x];
      rows[threadIdx.x] = (r >= 0 && r < n_rows) ? r : -1;
      gts[threadIdx.x] = gate[static_cast<size_t>(t) * K + threadIdx.x];
    }
    __syncthreads();
    for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
      float acc[8], x[8];
      if constexpr (KT > 0) {
        int rk[KT];
        uint4 vy[KT];
        const uint4 vu = ld_bf16x8(u, static_cast<size_t>(t) * d + c);
        const uint4 vs = ld_bf16x8(ysh, static_cast<size_t>(t) * d + c);   // Ns == 1 on this path
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          rk[k] = rows[k];
          vy[k] = rk[k] >= 0 ? ld_bf16x8(y, static_cast<size_t>(rk[k]) * d + c) : uint4{0, 0, 0, 0};
        }
        unpack_bf16x8(vu, acc);
        unpack_bf16x8(vs, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[i];
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          if (rk[k] < 0) continue;
          const float g = gts[k];
          unpack_bf16x8(vy[k], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, x[i], acc[i]);
        }
      } else {
        ld8(u, io, static_cast<size_t>(t) * d + c, acc);
        for (int sh = 0; sh < s.Ns; ++sh) {
          ld8(ysh, io, (static_cast<size_t>(sh) * s.T + t) * d + c, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += x[i];
        }
        for (int k = 0; k < K; ++k) {
          const int r = rows[k];
          if (r < 0) continue;
          const float g = gts[k];
          ld8(y, io, static_cast<size_t>(r) * d + c, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, x[i], acc[i]);
        }
      }
      const size_t o = static_cast<size_t>(t) * d + c;
      if (io == MOE_BF16) {
        uint4 v;
        v.x = pack_bf16x2(acc[0], acc[1]);
        v.y = pack_bf16x2(acc[2], acc[3]);
        v.z = pack_bf16x2(acc[4], acc[5]);
        v.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o) = v;
      } else {
        float* p = static_cast<float*>(out) + o;
        *reinterpret_cast<float4*>(p) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_combine(const Shape& s, moe_dtype io, const void* u, const void* y, const int32_t* row_of,
                          const float* gate, const void* ysh, void* out, hipStream_t st) {
  int threads = s.d / 8;
  if (threads > 1024) threads = 1024;
  threads = ((threads + 63) / 64) * 64;
  int blocks = s.T;
  const int cap = device_cu_count() * 32;
  if (blocks > cap) blocks = cap;
  const bool fast = io == MOE_BF16 && s.Ns == 1;
  if (fast && s.K == 8)
    hipLaunchKernelGGL(combine_kernel<8>, dim3(blocks), dim3(threads), 0, st, s, io, u, y, row_of, gate, ysh, out);
  else if (fast && s.K == 6)
    hipLaunchKernelGGL(combine_kernel<6>, dim3(blocks), dim3(threads), 0, st, s, io, u, y, row_of, gate, ysh, out);
  else
    hipLaunchKernelGGL(combine_kernel<0>, dim3(blocks), dim3(threads), 0, st, s, io, u, y, row_of, gate, ysh, out);
  return hipGetLastError();
}

// Overloaded (load > T*K/N_r): b -= gamma; underloaded: b += gamma; compared on integers.
__global__ void bias_update_kernel(int N, long long tk, const int32_t* __restrict__ load, float gamma,
                                   float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N) return;
  const long long scaled = static_cast<long long>(load[e]) * N;
  const float b = bias[e];
  if (scaled > tk) bias[e] = b - gamma;
  else if (scaled < tk) bias[e] = b + gamma;
}

hipError_t launch_bias_update(const Shape& s, const int32_t* load, float gamma, float* bias, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(cdiv(s.N, 256)), dim3(256), 0, st, s.N,
                     static_cast<long long>(s.T) * s.K, load, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
