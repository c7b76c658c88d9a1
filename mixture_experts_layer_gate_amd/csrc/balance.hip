// moe_balance_stats: the complementary sequence-wise balance statistics of
// eq. (17)-(20), "DeepSeek_V3_Report: Annotation", section "Complementary
// Sequence-Wise Auxiliary Loss": per run of seq_len tokens, the selection
// frequency f_i, the mean normalised affinity P_i and alpha * sum_i f_i P_i.
//
// Two passes, deterministic: chunks of 64 tokens of one sequence write their
// per-expert partial sums of s_{i,t} / sum_j s_{j,t} and their selection
// counts to the workspace; one block per sequence adds its chunks in order.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kBalChunk = 64;

static int bal_chunks_per_seq(int seq_len) { return cdiv(seq_len, kBalChunk); }

size_t balance_ws_bytes(const Shape& s, int seq_len) {
  const size_t n_seq = cdiv(s.T, seq_len);
  return n_seq * bal_chunks_per_seq(seq_len) * s.N * (sizeof(float) + sizeof(int32_t));
}

// One block (4 waves) per chunk; lane l owns experts l, l + 64, ... (V = N / 64 rounded up <= 16).
__global__ __launch_bounds__(256) void bal_partial_kernel(int T, int N, int K, int seq_len, int cps,
                                                          const float* __restrict__ scores,
                                                          const int32_t* __restrict__ idx, float* __restrict__ psum,
                                                          int32_t* __restrict__ pcnt) {
  __shared__ float part[4][1024];
  __shared__ int hist[1024];
  const int c = blockIdx.x, q = c / cps, j = c - q * cps;
  const int s0 = q * seq_len, s1 = min(T, s0 + seq_len);
  const int lo = min(s1, s0 + j * kBalChunk), hi = min(s1, lo + kBalChunk);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int t = lo + w; t < hi; t += 4) {
    const float* row = scores + static_cast<size_t>(t) * N;
    float x[16];
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int e = lane + 64 * v;
      x[v] = e < N ? row[e] : 0.0f;
      sum += x[v];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kWave);
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += x[v] / sum;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int e = lane + 64 * v;
    if (e < N) part[w][e] = acc[v];
  }
  for (int i = lo * K + threadIdx.x; i < hi * K; i += blockDim.x) {
    const int e = idx[i];
    if (e >= 0 && e < N) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    psum[static_cast<size_t>(c) * N + e] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
    pcnt[static_cast<size_t>(c) * N + e] = hist[e];
  }
}

// One block per sequence: chunks added in order, then the loss by a fixed-order tree.
__global__ __launch_bounds__(256) void bal_final_kernel(int T, int N, int K, int seq_len, int cps, float alpha,
                                                        const float* __restrict__ psum,
                                                        const int32_t* __restrict__ pcnt, float* __restrict__ f,
                                                        float* __restrict__ P, float* __restrict__ loss) {
  __shared__ float red[256];
  const int q = blockIdx.x;
  const int Ts = min(T, (q + 1) * seq_len) - q * seq_len;
  float mine = 0.0f;
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    float ps = 0.0f;
    int cnt = 0;
    for (int j = 0; j < cps; ++j) {
      const size_t o = static_cast<size_t>(q * cps + j) * N + e;
      ps += psum[o];
      cnt += pcnt[o];
    }
    const float fi = static_cast<float>(N) * static_cast<float>(cnt) / static_cast<float>(K * Ts);
    const float pi = ps / static_cast<float>(Ts);
    f[static_cast<size_t>(q) * N + e] = fi;
    P[static_cast<size_t>(q) * N + e] = pi;
    mine += fi * pi;
  }
  red[threadIdx.x] = mine;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[q] = alpha * red[0];
}

hipError_t launch_balance_stats(const Shape& s, const float* scores, const int32_t* idx, int seq_len, float alpha,
                                float* f, float* P, float* loss, void* ws, hipStream_t st) {
  const int cps = bal_chunks_per_seq(seq_len), n_seq = cdiv(s.T, seq_len);
  const int n_chunks = n_seq * cps;
  float* psum = static_cast<float*>(ws);
  int32_t* pcnt = reinterpret_cast<int32_t*>(psum + static_cast<size_t>(n_chunks) * s.N);
  hipLaunchKernelGGL(bal_partial_kernel, dim3(n_chunks), dim3(256), 0, st, s.T, s.N, s.K, seq_len, cps, scores, idx,
                     psum, pcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bal_final_kernel, dim3(n_seq), dim3(256), 0, st, s.T, s.N, s.K, seq_len, cps, alpha, psum, pcnt,
                     f, P, loss);
  return hipGetLastError();
}

}  // namespace moe
