// Grouped SwiGLU expert FFN in fp32 (the tiny fp32 workload) on the fp32
// matrix instruction v_mfma_f32_16x16x4_f32. One wave computes a 16-row x
// 16-column output tile of consecutive permuted rows; four waves of a block
// take four adjacent column tiles. The 16 rows may span several experts (the
// segments of the offsets), so the wave loops over the experts whose segment
// meets its rows and, for each, multiplies its rows masked to that expert
// (other rows contribute exact zeros) by that expert's weights. H (fp32
// [n_rows, I]) lives in the workspace.
//
// Operand layout of the 16x16x4 instruction: lane l supplies A[l % 16][k]
// and B[k][l % 16] for its k = l / 16 and receives C[4 (l / 16) + v][l % 16]
// in element v. Each lane loads four consecutive K values of its row and
// column (16-byte loads) and feeds them to four instructions, so one K chunk
// of 16 covers k0 + 4 (l / 16) + v.
#include "common.h"
#include "launch.h"
#include "sched.h"

namespace moe {

__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ off, int E, int n_rows, int r, int& seg0) {
  // last e with clamp(off[e]) <= r and r < clamp(off[e+1])
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (clampi(off[mid], 0, n_rows) <= r) lo = mid; else hi = mid;
  }
  seg0 = clampi(off[lo], 0, n_rows);
  const int s1 = clampi(off[lo + 1], seg0, n_rows);
  return (r >= seg0 && r < s1) ? lo : -1;
}

// Four consecutive values p[k .. k + 3] of a row of length K (zeros past K; p == nullptr: zeros).
__device__ __forceinline__ f32x4 load4(const float* __restrict__ p, int k, int K) {
  if (p == nullptr) return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if ((K & 3) == 0 && k + 4 <= K) return *reinterpret_cast<const f32x4*>(p + k);
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = k + q < K ? p[k + q] : 0.0f;
  return v;
}

__device__ __forceinline__ f32x4 mfma4(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
  for (int v = 0; v < 4; ++v) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[v], b[v], c, 0, 0, 0);
  return c;
}

// Experts whose clamped segment meets rows [r0, r1]: e_lo .. e_hi (inclusive; may include empty ones).
__device__ __forceinline__ void experts_of_rows(const int32_t* __restrict__ off, int E, int n_rows, int r0, int r1,
                                                int& e_lo, int& e_hi) {
  int s = 0;
  e_lo = expert_of_row(off, E, n_rows, r0, s);
  e_hi = expert_of_row(off, E, n_rows, r1, s);
  if (e_lo < 0 || e_hi < 0) {
    // a row outside every segment: scan the (few) experts for the ones that meet the range
    e_lo = E;
    e_hi = -1;
    for (int e = 0; e < E; ++e) {
      const int s0 = clampi(off[e], 0, n_rows), s1 = clampi(off[e + 1], s0, n_rows);
      if (s0 <= r1 && s1 > r0) {
        e_lo = min(e_lo, e);
        e_hi = e;
      }
    }
  }
}

__global__ __launch_bounds__(256) void ffn_gate_up_f32_kernel(int d, int I, int E, int n_rows, int a_rows,
                                                              const int32_t* __restrict__ off, moe_row_mode mode,
                                                              const int32_t* __restrict__ row_src,
                                                              const float* __restrict__ a,
                                                              const float* __restrict__ wgu, float* __restrict__ H) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 16, c0 = (blockIdx.y * 4 + w) * 16;
  if (c0 >= I) return;                                    // whole wave: no column of this tile exists
  const int r1 = min(r0 + 15, n_rows - 1);
  const int i = lane & 15, kq = 4 * (lane >> 4);
  const int r = r0 + i, c = c0 + i;                       // this lane's A row and B column
  f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f}, u = {0.0f, 0.0f, 0.0f, 0.0f};
  int e_lo, e_hi;
  experts_of_rows(off, E, n_rows, r0, r1, e_lo, e_hi);
  for (int e = e_lo; e <= e_hi; ++e) {
    const int s0 = clampi(off[e], 0, n_rows), s1 = clampi(off[e + 1], s0, n_rows);
    if (s0 > r1 || s1 <= r0) continue;
    const int sr = (r >= s0 && r < s1) ? source_row(mode, row_src, r, s0, a_rows) : -1;
    const float* x = sr >= 0 ? a + static_cast<size_t>(sr) * d : nullptr;
    const float* wg = c < I ? wgu + (static_cast<size_t>(e) * 2 * I + c) * d : nullptr;
    const float* wu = c < I ? wgu + (static_cast<size_t>(e) * 2 * I + I + c) * d : nullptr;
    for (int k0 = 0; k0 < d; k0 += 16) {
      const f32x4 xa = load4(x, k0 + kq, d);
      g = mfma4(xa, load4(wg, k0 + kq, d), g);
      u = mfma4(xa, load4(wu, k0 + kq, d), u);
    }
  }
  const int cc = c0 + (lane & 15);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = r0 + 4 * (lane >> 4) + v;
    if (rr < n_rows && cc < I) H[static_cast<size_t>(rr) * I + cc] = g[v] / (1.0f + expf(-g[v])) * u[v];
  }
}

__global__ __launch_bounds__(256) void ffn_down_f32_kernel(int d, int I, int E, int n_rows,
                                                           const int32_t* __restrict__ off,
                                                           const float* __restrict__ H, const float* __restrict__ wd,
                                                           moe_dtype ydt, void* __restrict__ y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 16, n0 = (blockIdx.y * 4 + w) * 16;
  if (n0 >= d) return;
  const int r1 = min(r0 + 15, n_rows - 1);
  const int i = lane & 15, kq = 4 * (lane >> 4);
  const int r = r0 + i, n = n0 + i;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int e_lo, e_hi;
  experts_of_rows(off, E, n_rows, r0, r1, e_lo, e_hi);
  for (int e = e_lo; e <= e_hi; ++e) {
    const int s0 = clampi(off[e], 0, n_rows), s1 = clampi(off[e + 1], s0, n_rows);
    if (s0 > r1 || s1 <= r0) continue;
    const float* h = (r >= s0 && r < s1) ? H + static_cast<size_t>(r) * I : nullptr;
    const float* wr = n < d ? wd + (static_cast<size_t>(e) * d + n) * I : nullptr;
    for (int k0 = 0; k0 < I; k0 += 16) acc = mfma4(load4(h, k0 + kq, I), load4(wr, k0 + kq, I), acc);
  }
  const int nn = n0 + (lane & 15);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = r0 + 4 * (lane >> 4) + v;
    if (rr >= n_rows || nn >= d) continue;
    int seg0 = 0;
    if (expert_of_row(off, E, n_rows, rr, seg0) < 0) continue;   // rows outside every segment are left as they are
    if (ydt == MOE_BF16) static_cast<uint16_t*>(y)[static_cast<size_t>(rr) * d + nn] = f32_to_bf16(acc[v]);
    else static_cast<float*>(y)[static_cast<size_t>(rr) * d + nn] = acc[v];
  }
}

hipError_t launch_ffn_f32_gate_up(const FfnArgs& p, hipStream_t st) {
  if (p.n_rows <= 0) return hipSuccess;
  dim3 g1(cdiv(p.n_rows, 16), cdiv(p.I, 64));
  hipLaunchKernelGGL(ffn_gate_up_f32_kernel, g1, dim3(256), 0, st, p.d, p.I, p.n_experts, p.n_rows, p.a_rows,
                     p.offsets, p.mode, p.row_src, static_cast<const float*>(p.a), static_cast<const float*>(p.w_gu),
                     static_cast<float*>(p.h));
  return hipGetLastError();
}

hipError_t launch_ffn_f32_down(const FfnArgs& p, hipStream_t st) {
  if (p.n_rows <= 0) return hipSuccess;
  dim3 g2(cdiv(p.n_rows, 16), cdiv(p.d, 64));
  hipLaunchKernelGGL(ffn_down_f32_kernel, g2, dim3(256), 0, st, p.d, p.I, p.n_experts, p.n_rows, p.offsets,
                     static_cast<const float*>(p.h), static_cast<const float*>(p.w_d), p.y_dtype, p.y);
  return hipGetLastError();
}

}  // namespace moe
