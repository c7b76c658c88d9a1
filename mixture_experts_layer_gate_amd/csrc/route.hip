// moe_route kernels: router logits GEMM with the sigmoid affinity epilogue
// (eq. (15) of "DeepSeek_V3_Report: Annotation"), then one wavefront per token
// for the biased, group-limited top-K selection (eq. (16) and the section
// "Node-Limited Routing"), the gates over the raw affinities (eq. (13)-(14))
// and the expert-load histogram that drives the step-end bias update.
#include <float.h>
#include <limits.h>

#include <mutex>

#include "common.h"
#include "gemm_pipe.h"
#include "gemm_w8.h"
#include "launch.h"
#include "sched.h"

namespace moe {

// ---------------------------------------------------------------- logits
// u . e_i for bf16 operands: the pipelined main loop of the expert GEMMs
// (gemm_pipe.h) on tiles of 256 centroids x 128 tokens, with K split into S
// slices so that a V3-sized batch fills every CU (64 token tiles x 4 slices).
// Slice s writes fp32 partial sums part[s][t][e]; the selection kernel adds the
// S partials in slice order and applies the sigmoid. Centroid rows past N and
// token rows past T read a valid row and are never stored.
using RouteTile = Pipe<256, 128>;

__global__ __launch_bounds__(RouteTile::NT, 1) void route_logits_bf16_kernel(
    int T, int d, int N, int n_wt, int kslice, int t_begin, int t_count, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ cent, float* __restrict__ part, int32_t* __restrict__ load) {
  using P = RouteTile;
  extern __shared__ __align__(16) uint8_t lds_route[];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && t_begin == 0)
    for (int e = tid; e < N; e += P::NT) load[e] = 0;   // histogram is rebuilt by the select kernel
  const int S = cdiv(d, kslice);
  const int ks = blockIdx.x % S, tile = blockIdx.x / S;
  const int w0 = (tile % n_wt) * P::BW, t0 = (tile / n_wt) * P::BT;   // t0 within this launch's token range
  const int k0 = ks * kslice, K = min(kslice, d - k0);
  PipeRows<P> rows;
  rows.wrs = pipe_rsrc(cent + k0, (static_cast<uint64_t>(N) * d - k0) * 2);
  rows.trs = pipe_rsrc(u + static_cast<size_t>(t_begin) * d + k0, (static_cast<uint64_t>(t_count) * d - k0) * 2);
#pragma unroll
  for (int q = 0; q < P::WL; ++q)
    rows.ow[q] = static_cast<uint32_t>(min(w0 + pipe_load_row(q), N - 1)) * d * 2 + pipe_load_chunk(q) * 16;
#pragma unroll
  for (int q = 0; q < P::TL; ++q)
    rows.ot[q] = static_cast<uint32_t>(min(t0 + pipe_load_row(q), t_count - 1)) * d * 2 + pipe_load_chunk(q) * 16;
  f32x16 acc[P::TW][P::TT];
#pragma unroll
  for (int j = 0; j < P::TW; ++j)
#pragma unroll
    for (int i = 0; i < P::TT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  pipe_mainloop<P, P::TT, P::TL>(rows, K, lds_route, acc);
#pragma unroll
  for (int i = 0; i < P::TT; ++i) {
    const int t = t0 + pipe_token_row(i);
    if (t >= t_count) continue;
    float* prow = part + (static_cast<size_t>(ks) * T + t_begin + t) * N;
#pragma unroll
    for (int j = 0; j < P::TW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = w0 + pipe_wcol<P>(j, q);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < N) prow[e + r] = acc[j][i][4 * q + r];
      }
  }
}

// The same product on the eight-wave loop of the expert GEMMs (gemm_w8.h),
// for N % 4 == 0: tiles of 256 centroids x 256 tokens (eight 32-row token
// sub-tiles of the loop's ten), K split into S slices of whole 128-wide
// chunks. At the V3 shape that is 32 token tiles x 8 slices, one per CU, each
// streaming 0.92 MB (the 128-token tiles above: 1.38 MB) at the loop's
// per-CU rate. Wave quarter ww holds centroids 64 ww .. 64 ww + 63 of the
// tile; each lane stores four consecutive partial sums of one token.
using RouteW8 = W8<false>;
constexpr int kRouteW8Tokens = 256;

template <int MS, int LT>
__device__ __forceinline__ void route_w8_tile(const W8Rows& rows, int K, uint8_t* lds, int T, int N, int w0, int t0,
                                              int t_count, int t_begin, int ks, float* __restrict__ part) {
  f32x16 acc[2][5];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  const int ww = wave_uniform((w8_tid() >> 6) & 3);
  const W8Offs o = w8_offsets(64 * ww, 64 * ww + 32);
  w8_mainloop<RouteW8, MS, LT>(rows, K, lds, o, acc);
  const int tid = w8_tid(), h = (tid & 63) >> 5;
  // rows t0 .. t_count - 1 of this launch's token range; a store past N or t_count is dropped by the range check
  const int rows_here = min(kRouteW8Tokens, t_count - t0);
  const __amdgpu_buffer_rsrc_t r =
      pipe_rsrc(part + (static_cast<size_t>(ks) * T + t_begin + t0) * N, static_cast<uint64_t>(rows_here) * N * 4);
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int tr = w8_token_row(i, tid);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = w0 + 64 * ww + 32 * j + 8 * q + 4 * h;
        const uint32_t off = e < N ? static_cast<uint32_t>(tr * N + e) * 4 : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[j][i][4 * q]), __float_as_uint(acc[j][i][4 * q + 1]),
                  __float_as_uint(acc[j][i][4 * q + 2]), __float_as_uint(acc[j][i][4 * q + 3])},
            r, off, 0, 0);
      }
  }
}

__global__ __launch_bounds__(RouteW8::NT, 1) void route_logits_w8_kernel(
    int T, int d, int N, int n_wt, int kslice, int t_begin, int t_count, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ cent, float* __restrict__ part, int32_t* __restrict__ load) {
  extern __shared__ __align__(16) uint8_t lds_rw8[];
  if (blockIdx.x == 0 && t_begin == 0)
    for (int e = threadIdx.x; e < N; e += RouteW8::NT) load[e] = 0;   // histogram is rebuilt by the select kernel
  const int S = cdiv(d, kslice);
  const int ks = blockIdx.x % S, tile = blockIdx.x / S;
  const int w0 = (tile % n_wt) * RouteW8::BW, t0 = (tile / n_wt) * kRouteW8Tokens;
  const int k0 = ks * kslice, K = min(kslice, d - k0);
  const int rows_t = min(kRouteW8Tokens, t_count - t0), nsub = cdiv(rows_t, 32);
  const int tid = w8_tid();
  W8Rows rows;
  rows.wrs = pipe_rsrc(cent + k0, (static_cast<uint64_t>(N) * d - k0) * 2);
  rows.trs = pipe_rsrc(u + (static_cast<size_t>(t_begin) + t0) * d + k0, (static_cast<uint64_t>(rows_t) * d - k0) * 2);
#pragma unroll
  for (int q = 0; q < RouteW8::WL; ++q) {
    const int uu = w8_unit(q, tid);
    rows.ow[q] = static_cast<uint32_t>(min(w0 + w8_load_row(uu, tid), N - 1)) * d * 2 + w8_load_chunk(uu, tid) * 16;
  }
#pragma unroll
  for (int q = 0; q < RouteW8::TLMAX; ++q) {
    const int uu = w8_unit(q, tid);
    rows.ot[q] = static_cast<uint32_t>(min(w8_load_row(uu, tid), rows_t - 1)) * d * 2 + w8_load_chunk(uu, tid) * 16;
  }
#define RW8_CALL(MS, LT) route_w8_tile<MS, LT>(rows, K, lds_rw8, T, N, w0, t0, t_count, t_begin, ks, part)
  W8_DISPATCH(nsub, RW8_CALL);
#undef RW8_CALL
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

// Logits of this lane's V experts (e0 .. e0 + nv - 1, nv <= V) from the slice
// partials part[p * slice + off + v], added in slice order; the loads of four
// slices are issued together (past the last slice: none) so that the chain of
// adds does not wait on one load at a time.
template <int V>
__device__ __forceinline__ void sum_slices(const float* __restrict__ part, int S_part, size_t slice, size_t off,
                                           int nv, float (&x)[V]) {
#pragma unroll
  for (int v = 0; v < V; ++v) x[v] = 0.0f;
  for (int p = 0; p < S_part; p += 4) {
    float y[4][V];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int v = 0; v < V; ++v) y[q][v] = (p + q < S_part && v < nv) ? part[(p + q) * slice + off + v] : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (p + q < S_part) x[v] = (p + q == 0) ? y[q][v] : x[v] + y[q][v];
  }
}

constexpr int kSelWaves = 4;

// part != nullptr: S partial logit sums per token (slice-major), added in
// slice order, then s = Sigmoid(sum) is written to scores (unless scores is
// NULL); otherwise scores already holds the affinities.
__global__ __launch_bounds__(64 * kSelWaves) void route_select_kernel(Shape s, const float* __restrict__ part,
                                                                      int S_part, float* __restrict__ scores,
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
        float v;
        if (part) {
          float x[1];
          sum_slices<1>(part, S_part, static_cast<size_t>(s.T) * N, static_cast<size_t>(t) * N + e, 1, x);
          v = 1.0f / (1.0f + expf(-x[0]));
          if (scores) scores[static_cast<size_t>(t) * N + e] = v;
        } else {
          v = scores[static_cast<size_t>(t) * N + e];
        }
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

// The bf16 logits GEMM's tiling: the eight-wave kernel when N % 4 == 0
// (256-centroid x 256-token tiles), else the four-wave one (256 x 128), with
// K split into slices of whole 128-wide chunks so that the tiles times the
// slices give every CU one, at most 32 slices. Batch-invariant mode: a fixed
// slice count whatever T is, so each logit is the same sum of the same
// partials in the same order for any batch; it is what a V3-sized batch
// needs to fill the GPU (eight-wave: 32 token tiles x 8; four-wave: 64 x 4).
struct RoutePlan {
  bool w8;
  int bt;       // token rows per tile
  int kslice;   // K elements per slice
};

static RoutePlan route_plan(const Shape& s) {
  const bool w8 = s.N % 4 == 0;
  const int bt = w8 ? kRouteW8Tokens : RouteTile::BT;
  const int chunks = s.d / 128;
  int S = s.bi ? (w8 ? 8 : 4) : device_cu_count() / (cdiv(s.N, 256) * cdiv(s.T, bt));
  S = S < 1 ? 1 : (S > 32 ? 32 : S);
  S = S > chunks ? chunks : S;
  return {w8, bt, cdiv(chunks, S) * 128};
}

static int route_kslice(const Shape& s) { return route_plan(s).kslice; }

size_t route_ws_bytes(const Shape& s, moe_dtype act) {
  const size_t scores = (static_cast<size_t>(s.T) * s.N * sizeof(float) + 255) & ~static_cast<size_t>(255);
  if (act != MOE_BF16) return scores;
  const size_t S = cdiv(s.d, route_kslice(s));
  return scores + S * s.T * s.N * sizeof(float);
}

// Register form of the selection, for shapes where each lane can own V
// consecutive experts and a group is a power-of-two run of whole lanes
// (S % V == 0, S / V a power of two <= 64; or no group limit). One wavefront
// per token, no LDS staging: each lane keeps its V biased scores; the group
// score comes from a butterfly merge of the lanes' top-4 lists. The M kept
// groups and the K picks are each found as a threshold: a 32-step binary
// search on order-preserving integer keys of the fp32 values, counting with
// wave ballots, then the values above the threshold plus the lowest-index
// ones equal to it. Same choices as route_select_kernel (larger value first,
// then the lower index), with no cross-lane shuffles in the searches.
__device__ __forceinline__ void top4_insert(float v, float& a0, float& a1, float& a2, float& a3) {
  // insert into the descending list a0 >= a1 >= a2 >= a3 (the largest four
  // stay), as a min/max bubble: no branches, no indexed registers
  float t = fminf(a0, v);
  a0 = fmaxf(a0, v);
  const float t1 = fminf(a1, t);
  a1 = fmaxf(a1, t);
  const float t2 = fminf(a2, t1);
  a2 = fmaxf(a2, t1);
  a3 = fmaxf(a3, t2);
}

// Unsigned key with the order of the (non-NaN) fp32 values; 0 marks "absent".
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_popc(uint64_t m) { return __builtin_popcountll(m); }

// Largest key t with #{candidates with key >= t} >= need (need >= 1 and at
// least need candidates have a key > 0); keys[v] of this lane, 0 = absent.
template <int V>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&keys)[V], int need) {
  uint32_t t = 0;
#pragma unroll 1
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) cnt += wave_popc(__ballot(keys[v] >= c));
    if (cnt >= need) t = c;
  }
  return t;
}

// sel[v]: whether this lane's candidate v is among the `need` largest keys
// (ties at the threshold to the lower index lane * V + v).
template <int V>
__device__ __forceinline__ void select_top(const uint32_t (&keys)[V], int need, bool (&sel)[V]) {
  const uint32_t t = kth_key<V>(keys, need);
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int above = 0, ties_before = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    above += wave_popc(__ballot(keys[v] > t));
    ties_before += wave_popc(__ballot(keys[v] == t) & below);
  }
  int quota = need - above;                      // ties to take, in index order
  int rank = ties_before;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const bool tie = keys[v] == t && keys[v] != 0;
    sel[v] = keys[v] > t || (tie && rank < quota);
    rank += tie ? 1 : 0;
  }
}

template <int V>
__global__ __launch_bounds__(256) void route_select_reg_kernel(Shape s, const float* __restrict__ part, int S_part,
                                                               float* __restrict__ scores,
                                                               const float* __restrict__ bias,
                                                               int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int N = s.N, G = s.G, M = s.M, K = s.K, topn = s.topn;
  const int S = N / G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool grouped = G > 1 && M < G;
  const int lpg = grouped ? S / V : 64;          // lanes per group
  const int my_group = grouped ? lane / lpg : 0;
  const int e0 = lane * V;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  float b[V];
#pragma unroll
  for (int v = 0; v < V; ++v) b[v] = e0 + v < N ? bias[e0 + v] : 0.0f;

  for (int t = blockIdx.x * 4 + w; t < s.T; t += gridDim.x * 4) {
    float sr[V], sb[V], lg[V];
    if (part)
      sum_slices<V>(part, S_part, static_cast<size_t>(s.T) * N, static_cast<size_t>(t) * N + e0, N - e0, lg);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = e0 + v;
      if (e < N) {
        float x;
        if (part) {
          x = 1.0f / (1.0f + expf(-lg[v]));
          if (scores) scores[static_cast<size_t>(t) * N + e] = x;
        } else {
          x = scores[static_cast<size_t>(t) * N + e];
        }
        sr[v] = x;
        sb[v] = x + b[v];
      } else {
        sr[v] = 0.0f;
        sb[v] = -INFINITY;
      }
    }
    bool live = true;                              // this lane's group is kept
    if (grouped) {
      float a0 = -INFINITY, a1 = -INFINITY, a2 = -INFINITY, a3 = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v) top4_insert(sb[v], a0, a1, a2, a3);
      for (int o = 1; o < lpg; o <<= 1) {
        const float c0 = __shfl_xor(a0, o, kWave), c1 = __shfl_xor(a1, o, kWave);
        const float c2 = __shfl_xor(a2, o, kWave), c3 = __shfl_xor(a3, o, kWave);
        top4_insert(c0, a0, a1, a2, a3);
        top4_insert(c1, a0, a1, a2, a3);
        top4_insert(c2, a0, a1, a2, a3);
        top4_insert(c3, a0, a1, a2, a3);
      }
      float gs = a0;                                 // summed from the largest down, in fp32
      if (topn > 1) gs = gs + a1;
      if (topn > 2) gs = gs + a2;
      if (topn > 3) gs = gs + a3;
      // one candidate per group: its first lane
      const uint32_t gk[1] = {(my_group < G && (lane % lpg) == 0) ? order_key(gs) : 0u};
      bool gsel[1];
      select_top<1>(gk, M, gsel);
      const uint64_t kept = __ballot(gsel[0]);
      live = my_group < G && ((kept >> (my_group * lpg)) & 1ull);
    }
    uint32_t keys[V];
#pragma unroll
    for (int v = 0; v < V; ++v) keys[v] = (live && e0 + v < N) ? order_key(sb[v]) : 0u;
    bool sel[V];
    select_top<V>(keys, K, sel);
    // slots in ascending expert order; gates over the raw affinities of the picks
    int before = 0;
    float part_sum = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      before += wave_popc(__ballot(sel[v]) & below);
      part_sum += sel[v] ? sr[v] : 0.0f;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part_sum += __shfl_xor(part_sum, o, kWave);
    int slot = before;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (sel[v]) {
        idx[static_cast<size_t>(t) * K + slot] = e0 + v;
        gate[static_cast<size_t>(t) * K + slot] = sr[v] / part_sum;
        ++slot;
      }
  }
}

// Expert-load histogram of the selections: a few blocks, each an LDS
// histogram of a contiguous run of topk_idx, added into load (zeroed by the
// logits kernel) -- one global atomic per expert and block.
__global__ __launch_bounds__(1024) void route_hist_kernel(long long n, int N, const int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ load) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const long long lo = n * blockIdx.x / gridDim.x, hi = n * (blockIdx.x + 1) / gridDim.x;
  for (long long i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    const int e = idx[i];
    if (e >= 0 && e < N) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    const int c = hist[e];
    if (c) atomicAdd(&load[e], c);
  }
}

// Experts per lane for the register selection, or 0 when the shape needs the
// LDS form.
static int select_lanes_v(const Shape& s) {
  const bool grouped = s.G > 1 && s.M < s.G;
  const int S = s.N / s.G;
  for (int V = cdiv(s.N, 64); V <= 16; ++V) {
    if (!grouped) return V;
    if (S % V) continue;
    const int lpg = S / V;
    if (lpg <= 64 && (lpg & (lpg - 1)) == 0) return V;
  }
  return 0;
}

template <int V>
static hipError_t launch_select_reg(const Shape& s, const float* part, int S, float* scores, const float* bias,
                                    int32_t* idx, float* gate, int32_t* load, hipStream_t st) {
  int blocks = cdiv(s.T, 4);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(route_select_reg_kernel<V>, dim3(blocks), dim3(256), 0, st, s, part, S, scores, bias, idx, gate);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = static_cast<long long>(s.T) * s.K;
  long long hb = (n + 1023) / 1024;               // about 1024 pairs per block: one pass of the block
  hb = hb < 1 ? 1 : (hb > 64 ? 64 : hb);
  hipLaunchKernelGGL(route_hist_kernel, dim3(static_cast<unsigned>(hb)), dim3(1024), 0, st, n, s.N, idx, load);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, moe_dtype act, const void* u, const void* cent, const float* bias,
                        int32_t* idx, float* gate, int32_t* load, float* scores, void* ws, hipStream_t st) {
  const float* part = nullptr;
  int S = 0;
  if (act == MOE_BF16) {
    const RoutePlan plan = route_plan(s);
    const int kslice = plan.kslice;
    S = cdiv(s.d, kslice);
    float* p = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                        ((static_cast<size_t>(s.T) * s.N * sizeof(float) + 255) & ~static_cast<size_t>(255)));
    part = p;
    static std::once_flag once;
    std::call_once(once, [] {
      // a refused request must not leave a sticky error
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(route_logits_bf16_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, RouteTile::LDS_BYTES);
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(route_logits_w8_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, RouteW8::LDS_BYTES);
      (void)hipGetLastError();
    });
    const int n_wt = cdiv(s.N, 256);
    // token ranges whose rows span less than 4 GiB (32-bit buffer offsets)
    const long long max_t = ((1LL << 32) - 1) / (2LL * s.d);
    const int t_step = static_cast<int>(max_t < s.T ? (max_t / plan.bt) * plan.bt : s.T);
    for (int t_begin = 0; t_begin < s.T; t_begin += t_step) {
      const int t_count = s.T - t_begin < t_step ? s.T - t_begin : t_step;
      const int grid = n_wt * cdiv(t_count, plan.bt) * S;
      if (plan.w8)
        hipLaunchKernelGGL(route_logits_w8_kernel, dim3(grid), dim3(RouteW8::NT), RouteW8::LDS_BYTES, st, s.T, s.d,
                           s.N, n_wt, kslice, t_begin, t_count, static_cast<const uint16_t*>(u),
                           static_cast<const uint16_t*>(cent), p, load);
      else
        hipLaunchKernelGGL(route_logits_bf16_kernel, dim3(grid), dim3(RouteTile::NT), RouteTile::LDS_BYTES, st, s.T,
                           s.d, s.N, n_wt, kslice, t_begin, t_count, static_cast<const uint16_t*>(u),
                           static_cast<const uint16_t*>(cent), p, load);
    }
  } else {
    dim3 grid(cdiv(s.N, 16), cdiv(s.T, 16));
    hipLaunchKernelGGL(route_logits_f32_kernel, grid, dim3(256), 0, st, s.T, s.d, s.N,
                       static_cast<const float*>(u), static_cast<const float*>(cent), scores, load);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (select_lanes_v(s)) {
#define MOE_SEL_CASE(V) \
  case V: return launch_select_reg<V>(s, part, S, scores, bias, idx, gate, load, st);
    MOE_SEL_CASE(1) MOE_SEL_CASE(2) MOE_SEL_CASE(3) MOE_SEL_CASE(4) MOE_SEL_CASE(5) MOE_SEL_CASE(6)
    MOE_SEL_CASE(7) MOE_SEL_CASE(8) MOE_SEL_CASE(9) MOE_SEL_CASE(10) MOE_SEL_CASE(11) MOE_SEL_CASE(12)
    MOE_SEL_CASE(13) MOE_SEL_CASE(14) MOE_SEL_CASE(15) MOE_SEL_CASE(16)
#undef MOE_SEL_CASE
    default: break;
  }
  const size_t lds = sizeof(float) * (static_cast<size_t>(s.N) + 2 * kSelWaves * static_cast<size_t>(s.N));
  int blocks = cdiv(s.T, kSelWaves);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(route_select_kernel, dim3(blocks), dim3(64 * kSelWaves), lds, st, s, part, S, scores, bias, idx,
                     gate, load);
  return hipGetLastError();
}

}  // namespace moe
