// moe_permute kernels: a deterministic stable counting sort of the T*K
// token-expert pairs by expert (every pair kept, section "No Token-Dropping"
// of "DeepSeek_V3_Report: Annotation"), and the row copy / online 1x128 fp8
// quantisation of activations (sections "Fine-Grained Quantization" and
// "Online Quantization").
//
// Sort in three passes over chunks of 64 tokens (one wavefront each):
//  1. mask[c][e] = bit set of the chunk's tokens that selected expert e
//     (LDS atomicOr: the result does not depend on the order of the atomics);
//  2. one block: per-expert totals, exclusive scan -> offsets, and the base
//     row of every (chunk, expert);
//  3. row of pair (t, k) = base[c][e] + popcount(mask[c][e] below lane t).
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kChunk = 64;

size_t permute_ws_bytes(const Shape& s) {
  const size_t nch = static_cast<size_t>(cdiv(s.T, kChunk));
  return nch * s.N * (sizeof(uint64_t) + sizeof(int32_t)) + 256;
}

__global__ __launch_bounds__(256) void perm_mask_kernel(int T, int K, int N, const int32_t* __restrict__ idx,
                                                        unsigned long long* __restrict__ masks) {
  extern __shared__ __align__(16) unsigned long long lds_mask[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = cdiv(T, kChunk);
  const int c = blockIdx.x * 4 + w;
  unsigned long long* m = lds_mask + static_cast<size_t>(w) * N;
  for (int e = lane; e < N; e += kWave) m[e] = 0ull;
  __syncthreads();
  const int t = c * kChunk + lane;
  if (c < nch && t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = idx[static_cast<size_t>(t) * K + k];
      if (e >= 0 && e < N) atomicOr(&m[e], 1ull << lane);
    }
  }
  __syncthreads();
  if (c < nch)
    for (int e = lane; e < N; e += kWave) masks[static_cast<size_t>(c) * N + e] = m[e];
}

constexpr int kScanRegs = 32;

// One block of 1024 threads. Thread (p, e) = (tid / N, tid % N) counts expert
// e's pairs over the p-th of P = 1024 / N runs of chunks (N <= 1024), so the
// chunk loop is P times shorter than with one thread per expert; the run
// sums give each run's start, and an exclusive scan of the expert totals
// gives the offsets.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int T, int N, const unsigned long long* __restrict__ masks,
                                                         int32_t* __restrict__ base, int32_t* __restrict__ offsets) {
  __shared__ int run_cnt[1024];
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int nch = cdiv(T, kChunk);
  const int P = 1024 / N;
  const int e = tid % N, p = tid / N;
  const bool act = p < P;
  const int c0 = act ? static_cast<int>(static_cast<long long>(p) * nch / P) : 0;
  const int c1 = act ? static_cast<int>(static_cast<long long>(p + 1) * nch / P) : 0;
  // runs of at most kScanRegs chunks (T <= 8192 with 256 experts): the run's masks are loaded together and
  // their counts kept in registers for the base pass; longer runs stream them twice
  const int n_run = c1 - c0;
  const bool in_regs = n_run <= kScanRegs;
  int pc[kScanRegs];
  int cnt = 0;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) pc[i] = i < n_run ? __popcll(masks[static_cast<size_t>(c0 + i) * N + e]) : 0;
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) cnt += pc[i];
  } else {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) cnt += __popcll(masks[static_cast<size_t>(c) * N + e]);
  }
  if (act) run_cnt[tid] = cnt;
  __syncthreads();
  // expert totals (threads e < N), then the exclusive scan over experts
  int total = 0;
  if (tid < N)
    for (int q = 0; q < P; ++q) total += run_cnt[q * N + tid];
  const int lane = tid & 63, w = tid >> 6;
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  const int excl = before + incl - total;
  if (tid < N) {
    offsets[tid] = excl;
    if (tid == N - 1) offsets[N] = excl + total;
    // start of run q of expert tid, written over its count
    int run = excl;
    for (int q = 0; q < P; ++q) {
      const int c = run_cnt[q * N + tid];
      run_cnt[q * N + tid] = run;
      run += c;
    }
  }
  __syncthreads();
  if (act) {
    int run = run_cnt[tid];
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kScanRegs; ++i)
        if (i < n_run) {
          base[static_cast<size_t>(c0 + i) * N + e] = run;
          run += pc[i];
        }
    } else {
#pragma unroll 8
      for (int c = c0; c < c1; ++c) {
        base[static_cast<size_t>(c) * N + e] = run;
        run += __popcll(masks[static_cast<size_t>(c) * N + e]);
      }
    }
  }
}

constexpr int kScatterK = 16;   // the largest top-K the library accepts

// A pair whose expert id is out of range or repeats an earlier id of the same
// token gets no row (row_of = -1); the masks count such a token once per
// distinct expert, so the rows past offsets[N] (their number) hold -1.
__global__ __launch_bounds__(256) void perm_scatter_kernel(int T, int K, int N, const int32_t* __restrict__ idx,
                                                           const unsigned long long* __restrict__ masks,
                                                           const int32_t* __restrict__ base,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ row_of) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = c * kChunk + lane;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* ti = idx + static_cast<size_t>(t) * K;
  if (K <= kScatterK) {
    // the token's ids, then the base and mask of every kept pair, each batch of loads issued together
    int ev[kScatterK];
#pragma unroll
    for (int k = 0; k < kScatterK; ++k) ev[k] = k < K ? ti[k] : -1;
    bool ok[kScatterK];
#pragma unroll
    for (int k = 0; k < kScatterK; ++k) {
      ok[k] = k < K && ev[k] >= 0 && ev[k] < N;
#pragma unroll
      for (int j = 0; j < k; ++j) ok[k] = ok[k] && ev[j] != ev[k];
    }
    int bv[kScatterK];
    unsigned long long mv[kScatterK];
#pragma unroll
    for (int k = 0; k < kScatterK; ++k) {
      const size_t ce = static_cast<size_t>(c) * N + (ok[k] ? ev[k] : 0);
      bv[k] = ok[k] ? base[ce] : 0;
      mv[k] = ok[k] ? masks[ce] : 0ull;
    }
#pragma unroll
    for (int k = 0; k < kScatterK; ++k) {
      if (k >= K) break;
      int r = -1;
      if (ok[k]) {
        r = bv[k] + __popcll(mv[k] & below);
        perm[r] = t;
      }
      row_of[static_cast<size_t>(t) * K + k] = r;
    }
  } else {
    for (int k = 0; k < K; ++k) {
      const int e = ti[k];
      bool ok = e >= 0 && e < N;
      for (int j = 0; j < k && ok; ++j) ok = ti[j] != e;
      if (!ok) {
        row_of[static_cast<size_t>(t) * K + k] = -1;
        continue;
      }
      const size_t ce = static_cast<size_t>(c) * N + e;
      const int r = base[ce] + __popcll(masks[ce] & below);
      perm[r] = t;
      row_of[static_cast<size_t>(t) * K + k] = r;
    }
  }
  const long long used = offsets[N];
  for (int k = 0; k < K; ++k) {
    const long long pos = static_cast<long long>(t) * K + k;
    if (pos >= used) perm[pos] = -1;
  }
}

hipError_t launch_permute_maps(const Shape& s, const int32_t* idx, int32_t* offsets, int32_t* perm,
                               int32_t* row_of, void* ws, hipStream_t st) {
  const int nch = cdiv(s.T, kChunk);
  auto* masks = static_cast<unsigned long long*>(ws);
  auto* base = reinterpret_cast<int32_t*>(masks + static_cast<size_t>(nch) * s.N);
  const int blocks = cdiv(nch, 4);
  hipLaunchKernelGGL(perm_mask_kernel, dim3(blocks), dim3(256), 4 * s.N * sizeof(unsigned long long), st, s.T, s.K,
                     s.N, idx, masks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, s.T, s.N, masks, base, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(blocks), dim3(256), 0, st, s.T, s.K, s.N, idx, masks, base, offsets,
                     perm, row_of);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row copy / quantise
// Sixteen lanes per 128-wide tile, eight elements per lane; a block of 256
// threads covers 16 tiles. Row r reads src[index[r]] (or src[r]).
__device__ __forceinline__ void load8(const void* src, moe_dtype dt, size_t off, float (&x)[8]) {
  if (dt == MOE_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

__global__ __launch_bounds__(256) void rows_copy_kernel(int n_rows, int d, moe_dtype sdt, const void* __restrict__ src,
                                                        int src_rows, const int32_t* __restrict__ index,
                                                        moe_dtype ddt, void* __restrict__ dst,
                                                        float* __restrict__ dscale) {
  const int tiles_per_row = d / 128;
  const long long total = static_cast<long long>(n_rows) * tiles_per_row;
  const int sub = threadIdx.x & 15;
  for (long long tile = static_cast<long long>(blockIdx.x) * 16 + (threadIdx.x >> 4); tile < total;
       tile += static_cast<long long>(gridDim.x) * 16) {
    const int r = static_cast<int>(tile / tiles_per_row);
    const int c = static_cast<int>(tile % tiles_per_row);
    const int sr = index ? index[r] : r;
    const bool ok = sr >= 0 && sr < src_rows;
    float x[8];
    if (ok) {
      load8(src, sdt, static_cast<size_t>(sr) * d + c * 128 + sub * 8, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0f;
    }
    const size_t doff = static_cast<size_t>(r) * d + c * 128 + sub * 8;
    if (ddt == MOE_F8E4M3 || ddt == MOE_F8E4M3_POW2) {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(x[i]));
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
      float scale = 1.0f;
      uint32_t lo = 0, hi = 0;
      if (ddt == MOE_F8E4M3) {
        const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
        lo = f32x4_to_e4m3(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
        hi = f32x4_to_e4m3(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
        if (amax > 0.0f) scale = amax / kE4M3Max;
      } else if (amax > 0.0f) {
        // scale = 2^n, the smallest power of two >= fl32(amax / 448); x * 2^-n is exact (ldexp), so
        // the codes are the encode of x / scale with no second rounding
        int e;
        const float m = __builtin_frexpf(amax / kE4M3Max, &e);  // v = m 2^e, 0.5 <= m < 1
        const int n = m == 0.5f ? e - 1 : e;
        scale = __builtin_ldexpf(1.0f, n);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = __builtin_ldexpf(x[i], -n);
        lo = f32x4_to_e4m3(y[0], y[1], y[2], y[3]);
        hi = f32x4_to_e4m3(y[4], y[5], y[6], y[7]);
      }
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(dst) + doff) = make_uint2(lo, hi);
      if (sub == 0) dscale[static_cast<size_t>(r) * tiles_per_row + c] = scale;
    } else if (ddt == MOE_BF16) {
      uint4 v;
      v.x = pack_bf16x2(x[0], x[1]);
      v.y = pack_bf16x2(x[2], x[3]);
      v.z = pack_bf16x2(x[4], x[5]);
      v.w = pack_bf16x2(x[6], x[7]);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + doff) = v;
    } else {
      float* o = static_cast<float*>(dst) + doff;
      *reinterpret_cast<float4*>(o) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
}

hipError_t launch_rows_copy(int n_rows, int d, moe_dtype src_dtype, const void* src, int src_rows,
                            const int32_t* index, moe_dtype dst_dtype, void* dst, float* dst_scale,
                            hipStream_t st) {
  const long long tiles = static_cast<long long>(n_rows) * (d / 128);
  long long blocks = (tiles + 15) / 16;
  const long long cap = static_cast<long long>(device_cu_count()) * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(rows_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, n_rows, d, src_dtype,
                     src, src_rows, index, dst_dtype, dst, dst_scale);
  return hipGetLastError();
}

}  // namespace moe
