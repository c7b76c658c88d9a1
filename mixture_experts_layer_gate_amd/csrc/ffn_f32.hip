// Grouped SwiGLU expert FFN in fp32 (the tiny fp32 workload). Every output
// element is one fp32 dot product; rows find their expert by a binary search
// over the offsets. H (fp32 [n_rows, I]) lives in the workspace.
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

__global__ __launch_bounds__(256) void ffn_gate_up_f32_kernel(int d, int I, int E, int n_rows, int a_rows,
                                                              const int32_t* __restrict__ off, moe_row_mode mode,
                                                              const int32_t* __restrict__ row_src,
                                                              const float* __restrict__ a,
                                                              const float* __restrict__ wgu, float* __restrict__ H) {
  const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = blockIdx.y * 16 + (threadIdx.x & 15);
  if (r >= n_rows || c >= I) return;
  int seg0 = 0;
  const int e = expert_of_row(off, E, n_rows, r, seg0);
  float h = 0.0f;
  if (e >= 0) {
    const int sr = source_row(mode, row_src, r, seg0, a_rows);
    if (sr >= 0) {
      const float* x = a + static_cast<size_t>(sr) * d;
      const float* wg = wgu + (static_cast<size_t>(e) * 2 * I + c) * d;
      const float* wu = wgu + (static_cast<size_t>(e) * 2 * I + I + c) * d;
      float g = 0.0f, up = 0.0f;
      for (int k = 0; k < d; ++k) {
        g = fmaf(x[k], wg[k], g);
        up = fmaf(x[k], wu[k], up);
      }
      h = g / (1.0f + expf(-g)) * up;
    }
  }
  H[static_cast<size_t>(r) * I + c] = h;
}

__global__ __launch_bounds__(256) void ffn_down_f32_kernel(int d, int I, int E, int n_rows,
                                                           const int32_t* __restrict__ off,
                                                           const float* __restrict__ H, const float* __restrict__ wd,
                                                           moe_dtype ydt, void* __restrict__ y) {
  const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int n = blockIdx.y * 16 + (threadIdx.x & 15);
  if (r >= n_rows || n >= d) return;
  int seg0 = 0;
  const int e = expert_of_row(off, E, n_rows, r, seg0);
  if (e < 0) return;
  const float* h = H + static_cast<size_t>(r) * I;
  const float* w = wd + (static_cast<size_t>(e) * d + n) * I;
  float acc = 0.0f;
  for (int k = 0; k < I; ++k) acc = fmaf(h[k], w[k], acc);
  if (ydt == MOE_BF16) static_cast<uint16_t*>(y)[static_cast<size_t>(r) * d + n] = f32_to_bf16(acc);
  else static_cast<float*>(y)[static_cast<size_t>(r) * d + n] = acc;
}

hipError_t launch_ffn_f32_gate_up(const FfnArgs& p, hipStream_t st) {
  dim3 g1(cdiv(p.n_rows, 16), cdiv(p.I, 16));
  hipLaunchKernelGGL(ffn_gate_up_f32_kernel, g1, dim3(256), 0, st, p.d, p.I, p.n_experts, p.n_rows, p.a_rows,
                     p.offsets, p.mode, p.row_src, static_cast<const float*>(p.a), static_cast<const float*>(p.w_gu),
                     static_cast<float*>(p.h));
  return hipGetLastError();
}

hipError_t launch_ffn_f32_down(const FfnArgs& p, hipStream_t st) {
  dim3 g2(cdiv(p.n_rows, 16), cdiv(p.d, 16));
  hipLaunchKernelGGL(ffn_down_f32_kernel, g2, dim3(256), 0, st, p.d, p.I, p.n_experts, p.n_rows, p.offsets,
                     static_cast<const float*>(p.h), static_cast<const float*>(p.w_d), p.y_dtype, p.y);
  return hipGetLastError();
}

}  // namespace moe
