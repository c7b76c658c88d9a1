// Weight gradients of the grouped expert FFN ("DeepSeek_V3_Report: Annotation",
// FP8 framework: the weight-gradient GEMM of each linear layer, weight
// gradients kept in fp32):
//   C[e][m][n] = sum over the rows r of expert e of X[r][m] * Y[src(r)][n],
// the contraction running over the expert's ragged rows (dW_d = dy^T h,
// dW_gate_up = [dG | dU]^T a). bf16 operands, fp32 MFMA accumulation, fp32
// output; experts without rows get zeros.
//
// A workgroup per (expert, 128 x 128 output tile), four waves in a 2 x 2 grid
// of 64 x 64 (2 x 2 MFMA tiles of 32 x 32). The rows advance in chunks of 32:
// each thread loads 16 consecutive columns of one row of X and of Y and writes
// them transposed into LDS ([column][row], 32 rows + 8 pad per column, so a
// lane's 8 consecutive rows are one 16-byte read and 16 lanes hit 16
// different bank groups); two K16 MFMA steps per chunk. Rows past the expert's
// last are zero.
#include "common.h"
#include "launch.h"
#include "sched.h"

namespace moe {

constexpr int kWgTile = 128, kWgK = 32, kWgLd = kWgK + 8;

__global__ __launch_bounds__(256) void wgrad_kernel(int M, int N, int E, int n_rows, int a_rows,
                                                    const int32_t* __restrict__ off, moe_row_mode mode,
                                                    const int32_t* __restrict__ row_src,
                                                    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y,
                                                    float* __restrict__ C) {
  __shared__ __align__(16) uint16_t xs[kWgTile][kWgLd];
  __shared__ __align__(16) uint16_t ys[kWgTile][kWgLd];
  const int mt = M / kWgTile, nt = N / kWgTile;
  const long long b = blockIdx.x;
  const int e = static_cast<int>(b / (static_cast<long long>(mt) * nt));
  const int rem = static_cast<int>(b % (static_cast<long long>(mt) * nt));
  const int m0 = (rem / nt) * kWgTile, n0 = (rem % nt) * kWgTile;
  if (e >= E) return;
  const int lo = clampi(off[e], 0, n_rows), hi = clampi(off[e + 1], lo, n_rows);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, wm = w >> 1, wn = w & 1;
  const int kk = tid >> 3, cs = (tid & 7) * 16;       // the row and 16 columns this thread loads
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
  for (int r0 = lo; r0 < hi; r0 += kWgK) {
    const int r = r0 + kk;
    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0, y0 = x0, y1 = x0;
    if (r < hi) {
      const uint4* xp = reinterpret_cast<const uint4*>(X + static_cast<size_t>(r) * M + m0 + cs);
      x0 = xp[0];
      x1 = xp[1];
      const int sr = source_row(mode, row_src, r, lo, a_rows);
      if (sr >= 0) {
        const uint4* yp = reinterpret_cast<const uint4*>(Y + static_cast<size_t>(sr) * N + n0 + cs);
        y0 = yp[0];
        y1 = yp[1];
      }
    }
    __syncthreads();                                   // the previous chunk's fragments have been read
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t yw[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xs[cs + 2 * i][kk] = static_cast<uint16_t>(xw[i] & 0xFFFFu);
      xs[cs + 2 * i + 1][kk] = static_cast<uint16_t>(xw[i] >> 16);
      ys[cs + 2 * i][kk] = static_cast<uint16_t>(yw[i] & 0xFFFFu);
      ys[cs + 2 * i + 1][kk] = static_cast<uint16_t>(yw[i] >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int k = ks * 16 + 8 * (l >> 5);
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) fa[a] = *reinterpret_cast<const bf16x8*>(&xs[wm * 64 + a * 32 + (l & 31)][k]);
#pragma unroll
      for (int c = 0; c < 2; ++c) fb[c] = *reinterpret_cast<const bf16x8*>(&ys[wn * 64 + c * 32 + (l & 31)][k]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[a][c] = mfma_32x32x16_bf16(fa[a], fb[c], acc[a][c]);
    }
  }
  float* Ce = C + static_cast<size_t>(e) * M * N;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int n = n0 + wn * 64 + c * 32 + (l & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        Ce[static_cast<size_t>(m) * N + n] = acc[a][c][v];
      }
    }
}

hipError_t launch_wgrad(int M, int N, int E, int n_rows, int a_rows, const int32_t* off, moe_row_mode mode,
                        const int32_t* row_src, const void* X, const void* Y, float* C, hipStream_t st) {
  const long long blocks = static_cast<long long>(E) * (M / kWgTile) * (N / kWgTile);
  hipLaunchKernelGGL(wgrad_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, M, N, E, n_rows, a_rows, off,
                     mode, row_src, static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Y), C);
  return hipGetLastError();
}

}  // namespace moe
