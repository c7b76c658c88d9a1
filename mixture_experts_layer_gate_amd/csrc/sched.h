// Persistent grouped-GEMM schedule shared by the expert FFN kernels.
//
// Work unit = (expert e, n-block, m-block) with m-blocks of BM rows over the
// expert's ragged row segment [off[e], off[e+1]). Units are numbered expert by
// expert, n-block by n-block, m-block fastest, so consecutive units share the
// same weight tile (all m-blocks of one n-block) and the same expert.
// Units are handed out dynamically (unit_queue_next): the unit list is cut
// into 8 contiguous ranges, one per XCD (workgroups go to the 8 XCDs
// round-robin, so workgroup b runs on XCD b % 8), and a workgroup takes the
// next unit of its XCD's range with an atomic counter, then helps the other
// ranges. Runs of consecutive units -- one expert's weight and activation
// tiles -- stay inside one XCD's L2, and unequal units (ragged experts) no
// longer leave some CUs a whole unit behind the others.
#pragma once

#include "common.h"

namespace moe {

// In-place exclusive scan of a[0..n) in LDS, a[n] = total. Every thread of the
// block must call it.
__device__ __forceinline__ void block_exclusive_scan(int* a, int n, int* wtmp /* >= 16 ints */) {
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (n + nt - 1) / nt;
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += a[i];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wtmp[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wtmp[i];
  const int excl = before + incl - sum;
  int run = excl;
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  if (tid == nt - 1) a[n] = excl + sum;
  __syncthreads();
}

// The unit is the same for every lane (derived from the block index and LDS
// values read at uniform addresses); saying so keeps it in SGPRs.
__device__ __forceinline__ int wave_uniform(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(x);
#else
  return x;
#endif
}

struct Unit {
  int e, nb, m0, rows, seg0;  // expert, n-block, first row, valid rows (<= BM), segment start
  int nsub;                   // 32-row sub-tiles in this block (balanced schedule)
};

// Fill cum[0..E] (LDS) with units-before-expert; returns the total.
__device__ __forceinline__ int build_units(const int32_t* __restrict__ off, int E, int n_rows, int BM, int NB,
                                           int* cum, int* wtmp) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int lo = clampi(off[e], 0, n_rows);
    const int hi = clampi(off[e + 1], lo, n_rows);
    cum[e] = cdiv(hi - lo, BM) * NB;
  }
  __syncthreads();
  block_exclusive_scan(cum, E, wtmp);
  return cum[E];
}

__device__ __forceinline__ Unit find_unit(int t, const int32_t* __restrict__ off, int E, int n_rows, int BM,
                                          const int* cum) {
  int lo = 0, hi = E;  // largest e with cum[e] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] <= t) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int s0 = clampi(off[e], 0, n_rows);
  const int s1 = clampi(off[e + 1], s0, n_rows);
  const int nmb = cdiv(s1 - s0, BM);
  const int local = t - cum[e];
  Unit u;
  u.e = e;
  u.nb = local / nmb;
  u.m0 = s0 + (local % nmb) * BM;
  u.rows = min(BM, s1 - u.m0);
  u.seg0 = s0;
  return u;
}

// Blocks of an expert: its rows are cut into 32-row sub-tiles, and the
// sub-tiles into nmb = ceil(n32 / MAXSUB) blocks, either of nearly equal size
// (BALANCED: a 260-row expert becomes 2 x 130 rows; best for the bf16 tiles of
// 8 sub-tiles) or full blocks first and the remainder last (260 rows with 4
// sub-tiles per block: 128 + 128 + 4; best for the fp8 tiles, where a full
// block runs at full MFMA rate and a one-sub-tile block is cheap).
// Units are enumerated from the last expert down (cum[k] counts the units of
// experts E-1 .. E-k): the shared experts, appended after the routed ones and
// the largest, are handed out first and the routed tiles fill the tail.
__device__ __forceinline__ int build_units_balanced(const int32_t* __restrict__ off, int E, int n_rows, int MAXSUB,
                                                    int NB, int* cum, int* wtmp) {
  for (int k = threadIdx.x; k < E; k += blockDim.x) {
    const int e = E - 1 - k;
    const int lo = clampi(off[e], 0, n_rows);
    const int hi = clampi(off[e + 1], lo, n_rows);
    cum[k] = cdiv(cdiv(hi - lo, 32), MAXSUB) * NB;
  }
  __syncthreads();
  block_exclusive_scan(cum, E, wtmp);
  return cum[E];
}

template <bool BALANCED = true>
__device__ __forceinline__ Unit find_unit_balanced(int t, const int32_t* __restrict__ off, int E, int n_rows,
                                                   int MAXSUB, const int* cum) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] <= t) lo = mid; else hi = mid;
  }
  const int e = E - 1 - lo;
  const int s0 = clampi(off[e], 0, n_rows);
  const int s1 = clampi(off[e + 1], s0, n_rows);
  const int n32 = cdiv(s1 - s0, 32);
  const int nmb = cdiv(n32, MAXSUB);
  const int local = t - cum[lo];
  const int b = local % nmb;
  const int first = BALANCED ? b * n32 / nmb : b * MAXSUB;
  const int last = BALANCED ? (b + 1) * n32 / nmb : min(n32, (b + 1) * MAXSUB);
  Unit u;
  u.e = wave_uniform(e);
  u.nb = wave_uniform(local / nmb);
  u.m0 = wave_uniform(s0 + 32 * first);
  u.rows = wave_uniform(min(32 * (last - first), s1 - u.m0));
  u.seg0 = wave_uniform(s0);
  u.nsub = wave_uniform(last - first);
  return u;
}

__device__ __forceinline__ int xcd_virtual_block() {
  const int G = gridDim.x, b = blockIdx.x;
  return (b & 7) * (G >> 3) + (b >> 3);
}

// Counters of one launch: q[x] = units taken so far from XCD range x. They
// live in the caller's workspace and are zeroed (launch_queue_reset) on the
// same stream right before the launch.
constexpr int kQueueInts = 32;   // ints per launch (128 bytes)

// Next unit for this workgroup, or -1 when every range is exhausted. Every
// thread of the block calls it; x_off (the ranges this workgroup has
// exhausted) is only used by thread 0. slot: one int of shared memory.
__device__ __forceinline__ int unit_queue_next(int* __restrict__ q, int total, int& x_off, int* slot) {
  if (threadIdx.x == 0) {
    int t = -1;
    const int x0 = blockIdx.x & 7;
    while (x_off < 8) {
      const int x = (x0 + x_off) & 7;
      const int lo = static_cast<int>(static_cast<long long>(x) * total / 8);
      const int hi = static_cast<int>(static_cast<long long>(x + 1) * total / 8);
      if (lo < hi) {
        const int v = lo + atomicAdd(&q[x], 1);
        if (v < hi) {
          t = v;
          break;
        }
      }
      ++x_off;
    }
    *slot = t;
  }
  __syncthreads();
  const int t = wave_uniform(*slot);
  __syncthreads();
  return t;
}

// Index of the input row for output row r (absolute) of an expert whose segment starts at seg0.
__device__ __forceinline__ int source_row(moe_row_mode mode, const int32_t* __restrict__ row_src, int r, int seg0,
                                          int a_rows) {
  int s = r;
  if (mode == MOE_ROWS_GATHER) s = row_src[r];
  else if (mode == MOE_ROWS_SEGMENT) s = r - seg0;
  return (s >= 0 && s < a_rows) ? s : -1;
}

}  // namespace moe
