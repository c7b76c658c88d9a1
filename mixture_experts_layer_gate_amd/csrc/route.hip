// moe_route kernels: router logits GEMM with the sigmoid affinity epilogue
// (eq. (15) of "DeepSeek_V3_Report: Annotation"), then one wavefront per token
// for the biased, group-limited top-K selection (eq. (16) and the section
// "Node-Limited Routing"), the gates over the raw affinities (eq. (13)-(14))
// and the expert-load histogram that drives the step-end bias update.
#include <float.h>
#include <limits.h>

#include "common.h"
#include "gemm_bf16.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------- logits
// scores[t, e] = Sigmoid(u[t] . centroid[e]); bf16 operands, fp32 MFMA accumulation.
using RouteTile = TileBF16<64, 128, 2, 2>;

__global__ __launch_bounds__(RouteTile::NT) void route_logits_bf16_kernel(
    int T, int d, int N, const uint16_t* __restrict__ u, const uint16_t* __restrict__ cent,
    float* __restrict__ scores, int32_t* __restrict__ load) {
  using G = RouteTile;
  extern __shared__ __align__(16) uint16_t lds_route[];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < N; e += G::NT) load[e] = 0;   // histogram is rebuilt by the select kernel
  const int n0 = blockIdx.x * G::BN;
  const int m0 = blockIdx.y * G::BM;
  const uint16_t* pa[G::AC];
  const uint16_t* pb[G::BC];
#pragma unroll
  for (int j = 0; j < G::AC; ++j) {
    const int r = m0 + chunk_row<G>(tid, j);
    pa[j] = r < T ? u + static_cast<size_t>(r) * d + chunk_col<G>(tid, j) : nullptr;
  }
#pragma unroll
  for (int j = 0; j < G::BC; ++j) {
    const int e = n0 + chunk_row<G>(tid, j);
    pb[j] = e < N ? cent + static_cast<size_t>(e) * d + chunk_col<G>(tid, j) : nullptr;
  }
  f32x16 acc[G::TM][G::TN];
  zero_acc<G>(acc);
  mainloop_bf16<G>(pa, pb, d, lds_route, acc);
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) {
      const int e = n0 + acc_col<G>(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = m0 + acc_row<G>(i, v);
        if (t < T && e < N) scores[static_cast<size_t>(t) * N + e] = 1.0f / (1.0f + expf(-acc[i][j][v]));
      }
    }
}

// fp32 operands: 16x16 output tile per block, 16-wide K slices through LDS.
__global__ __launch_bounds__(256) void route_logits_f32_kernel(int T, int d, int N, const float* __restrict__ u,
                                                               const float* __restrict__ cent,
                                                               float* __restrict__ scores, int32_t* __restrict__ load) {
  __shared__ float su[16][17];
  __shared__ float se[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = threadIdx.x; e < N; e += 256) load[e] = 0;
  const int t = blockIdx.y * 16 + ty;
  const int e = blockIdx.x * 16 + tx;
  const int tl = blockIdx.y * 16 + tx;  // loader rows
  const int el = blockIdx.x * 16 + tx;
  float acc = 0.0f;
  for (int k0 = 0; k0 < d; k0 += 16) {
    su[ty][tx] = 0.0f;
    se[ty][tx] = 0.0f;
    const int tr = blockIdx.y * 16 + ty, er = blockIdx.x * 16 + ty;
    if (tr < T) su[ty][tx] = u[static_cast<size_t>(tr) * d + k0 + tx];
    if (er < N) se[ty][tx] = cent[static_cast<size_t>(er) * d + k0 + tx];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) acc = fmaf(su[ty][k], se[tx][k], acc);
    __syncthreads();
  }
  (void)tl;
  (void)el;
  if (t < T && e < N) scores[static_cast<size_t>(t) * N + e] = 1.0f / (1.0f + expf(-acc));
}

// ---------------------------------------------------------------- selection
// One wavefront per token. s' = fl32(s + b) staged in LDS; group scores by
// the lanes < G; M rounds of a wave argmax pick the groups, K rounds pick the
// experts. Ties: larger value first, then the lower index.
__device__ __forceinline__ void argmax_pair(float& v, int& id) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(id, o, kWave);
    if (ov > v || (ov == v && oi < id)) {
      v = ov;
      id = oi;
    }
  }
}

constexpr int kSelWaves = 4;

__global__ __launch_bounds__(64 * kSelWaves) void route_select_kernel(Shape s, const float* __restrict__ scores,
                                                                      const float* __restrict__ bias,
                                                                      int32_t* __restrict__ idx,
                                                                      float* __restrict__ gate,
                                                                      int32_t* __restrict__ load) {
  extern __shared__ __align__(16) float lds_sel[];
  const int N = s.N, G = s.G, M = s.M, K = s.K, topn = s.topn;
  const int S = N / G;
  int* hist = reinterpret_cast<int*>(lds_sel);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* sr = lds_sel + N + w * 2 * N;   // raw affinities of this wave's token
  float* sb = sr + N;                    // biased scores (removed entries set to -inf)
  const bool grouped = G > 1 && M < G;

  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  for (int t0 = blockIdx.x * kSelWaves; t0 < s.T; t0 += gridDim.x * kSelWaves) {
    const int t = t0 + w;
    const bool active = t < s.T;
    if (active) {
      for (int e = lane; e < N; e += kWave) {
        const float v = scores[static_cast<size_t>(t) * N + e];
        sr[e] = v;
        sb[e] = v + bias[e];
      }
    }
    __syncthreads();
    if (active) {
      uint64_t keep = ~0ull;
      if (grouped) {
        float gs = -INFINITY;
        if (lane < G) {
          float a0 = -INFINITY, a1 = -INFINITY, a2 = -INFINITY, a3 = -INFINITY;
          for (int i = 0; i < S; ++i) {
            const float v = sb[lane * S + i];
            if (v > a0) { a3 = a2; a2 = a1; a1 = a0; a0 = v; }
            else if (v > a1) { a3 = a2; a2 = a1; a1 = v; }
            else if (v > a2) { a3 = a2; a2 = v; }
            else if (v > a3) { a3 = v; }
          }
          gs = a0;                       // summed from the largest down, in fp32
          if (topn > 1) gs = gs + a1;
          if (topn > 2) gs = gs + a2;
          if (topn > 3) gs = gs + a3;
        }
        keep = 0ull;
        for (int m = 0; m < M; ++m) {
          float v = (lane < G && !((keep >> lane) & 1ull)) ? gs : -INFINITY;
          int id = lane < G && !((keep >> lane) & 1ull) ? lane : INT_MAX;
          argmax_pair(v, id);
          if (id < 64) keep |= 1ull << id;
        }
      }
      int my_pick = -1;
      for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int be = INT_MAX;
        for (int e = lane; e < N; e += kWave) {
          if (!((keep >> (e / S)) & 1ull)) continue;
          const float v = sb[e];
          if (v > bv) { bv = v; be = e; }
        }
        argmax_pair(bv, be);
        if (lane == k) my_pick = be < N ? be : -1;
        if (be < N && lane == (be & 63)) sb[be] = -INFINITY;
      }
      // ascending expert order; gates over the raw affinities of the picks
      int rank = 0;
      float my_s = 0.0f, sum = 0.0f;
      if (lane < K && my_pick >= 0) my_s = sr[my_pick];
      for (int j = 0; j < K; ++j) {
        const int pj = __shfl(my_pick, j, kWave);
        sum += __shfl(my_s, j, kWave);
        rank += (pj < my_pick) ? 1 : 0;
      }
      if (lane < K) {
        idx[static_cast<size_t>(t) * K + rank] = my_pick;
        gate[static_cast<size_t>(t) * K + rank] = my_s / sum;
        if (my_pick >= 0) atomicAdd(&hist[my_pick], 1);
      }
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    const int c = hist[e];
    if (c) atomicAdd(&load[e], c);
  }
}

hipError_t launch_route(const Shape& s, moe_dtype act, const void* u, const void* cent, const float* bias,
                        int32_t* idx, float* gate, int32_t* load, float* scores, hipStream_t st) {
  if (act == MOE_BF16) {
    using G = RouteTile;
    dim3 grid(cdiv(s.N, G::BN), cdiv(s.T, G::BM));
    hipLaunchKernelGGL(route_logits_bf16_kernel, grid, dim3(G::NT), G::LDS_BYTES, st, s.T, s.d, s.N,
                       static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(cent), scores, load);
  } else {
    dim3 grid(cdiv(s.N, 16), cdiv(s.T, 16));
    hipLaunchKernelGGL(route_logits_f32_kernel, grid, dim3(256), 0, st, s.T, s.d, s.N,
                       static_cast<const float*>(u), static_cast<const float*>(cent), scores, load);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) * (static_cast<size_t>(s.N) + 2 * kSelWaves * static_cast<size_t>(s.N));
  int blocks = cdiv(s.T, kSelWaves);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(route_select_kernel, dim3(blocks), dim3(64 * kSelWaves), lds, st, s, scores, bias, idx, gate,
                     load);
  return hipGetLastError();
}

}  // namespace moe
