// Grouped SwiGLU expert FFN in bf16 with fp32 MFMA accumulation
// ("DeepSeek_V3_Report: Annotation", SwiGLU paragraph and eq. (12)).
//
// Two persistent launches over all experts, 128 x 128 tiles, both operands
// staged through double-buffered LDS:
//  1. gate/up: H[r, c] = SiLU(x_r . Wg[c]) * (x_r . Wu[c]) for 64 H columns;
//     the B tile interleaves 32 gate rows and the matching 32 up rows per
//     wave, so the SwiGLU product is formed in registers. Input rows are read
//     through the row mode (the gather is fused into the A load).
//  2. down:    y[r, n] = H_r . Wd[n] for 128 output columns.
// H lives in the workspace as bf16 [n_rows, I].
#include <mutex>

#include "common.h"
#include "gemm_bf16.h"
#include "launch.h"
#include "sched.h"

namespace moe {

using FfnTile = TileBF16<128, 128, 2, 2>;
constexpr int kGuBNh = 64;  // H columns per gate/up tile

__global__ __launch_bounds__(FfnTile::NT) void ffn_gate_up_bf16_kernel(
    int d, int I, int E, int n_rows, int a_rows, const int32_t* __restrict__ off, moe_row_mode mode,
    const int32_t* __restrict__ row_src, const uint16_t* __restrict__ a, const uint16_t* __restrict__ wgu,
    uint16_t* __restrict__ H) {
  using G = FfnTile;
  extern __shared__ __align__(16) uint16_t lds_ffn[];
  int* cum = reinterpret_cast<int*>(lds_ffn + G::LDS_BYTES / 2);
  __shared__ int wtmp[16];
  const int NB = I / kGuBNh;
  const int total = build_units(off, E, n_rows, G::BM, NB, cum, wtmp);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = (tid >> 6) / G::WM;
  for (int t = xcd_virtual_block(); t < total; t += gridDim.x) {
    const Unit un = find_unit(t, off, E, n_rows, G::BM, cum);
    const uint16_t* pa[G::AC];
    const uint16_t* pb[G::BC];
#pragma unroll
    for (int j = 0; j < G::AC; ++j) {
      const int r = chunk_row<G>(tid, j);
      const int sr = r < un.rows ? source_row(mode, row_src, un.m0 + r, un.seg0, a_rows) : -1;
      pa[j] = sr >= 0 ? a + static_cast<size_t>(sr) * d + chunk_col<G>(tid, j) : nullptr;
    }
    // B tile rows: per wave column group wn, 32 gate rows then the matching 32 up rows
    const uint16_t* wexp = wgu + static_cast<size_t>(un.e) * 2 * I * d;
#pragma unroll
    for (int j = 0; j < G::BC; ++j) {
      const int rb = chunk_row<G>(tid, j);
      const int hcol = un.nb * kGuBNh + (rb >> 6) * 32 + (rb & 31);
      const int wrow = ((rb >> 5) & 1) ? I + hcol : hcol;
      pb[j] = wexp + static_cast<size_t>(wrow) * d + chunk_col<G>(tid, j);
    }
    f32x16 acc[G::TM][G::TN];
    zero_acc<G>(acc);
    mainloop_bf16<G>(pa, pb, d, lds_ffn, acc);
    const int col = un.nb * kGuBNh + wn * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = acc_row<G>(i, v);
        if (r < un.rows) {
          const float h = silu(acc[i][0][v]) * acc[i][1][v];
          H[static_cast<size_t>(un.m0 + r) * I + col] = f32_to_bf16(h);
        }
      }
  }
}

__global__ __launch_bounds__(FfnTile::NT) void ffn_down_bf16_kernel(int d, int I, int E, int n_rows,
                                                                    const int32_t* __restrict__ off,
                                                                    const uint16_t* __restrict__ H,
                                                                    const uint16_t* __restrict__ wd,
                                                                    uint16_t* __restrict__ y) {
  using G = FfnTile;
  extern __shared__ __align__(16) uint16_t lds_ffn[];
  int* cum = reinterpret_cast<int*>(lds_ffn + G::LDS_BYTES / 2);
  __shared__ int wtmp[16];
  const int NB = d / G::BN;
  const int total = build_units(off, E, n_rows, G::BM, NB, cum, wtmp);
  const int tid = threadIdx.x;
  for (int t = xcd_virtual_block(); t < total; t += gridDim.x) {
    const Unit un = find_unit(t, off, E, n_rows, G::BM, cum);
    const uint16_t* pa[G::AC];
    const uint16_t* pb[G::BC];
#pragma unroll
    for (int j = 0; j < G::AC; ++j) {
      const int r = chunk_row<G>(tid, j);
      pa[j] = r < un.rows ? H + static_cast<size_t>(un.m0 + r) * I + chunk_col<G>(tid, j) : nullptr;
    }
    const uint16_t* wexp = wd + static_cast<size_t>(un.e) * d * I;
#pragma unroll
    for (int j = 0; j < G::BC; ++j) {
      const int n = un.nb * G::BN + chunk_row<G>(tid, j);
      pb[j] = wexp + static_cast<size_t>(n) * I + chunk_col<G>(tid, j);
    }
    f32x16 acc[G::TM][G::TN];
    zero_acc<G>(acc);
    mainloop_bf16<G>(pa, pb, I, lds_ffn, acc);
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int n = un.nb * G::BN + acc_col<G>(j);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = acc_row<G>(i, v);
          if (r < un.rows) y[static_cast<size_t>(un.m0 + r) * d + n] = f32_to_bf16(acc[i][j][v]);
        }
      }
  }
}

static int persistent_grid(long long units_upper, int per_cu) {
  long long g = static_cast<long long>(device_cu_count()) * per_cu;
  if (units_upper < g) g = units_upper;
  g = ((g + 7) / 8) * 8;
  return static_cast<int>(g < 8 ? 8 : g);
}

static void set_lds_limits() {
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_gate_up_bf16_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_down_bf16_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  });
}

hipError_t launch_ffn_bf16_gate_up(const FfnArgs& p, hipStream_t st) {
  using G = FfnTile;
  set_lds_limits();
  const size_t lds = G::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / G::BM + p.n_experts;
  const int g1 = persistent_grid(mblocks * (p.I / kGuBNh), 2);
  hipLaunchKernelGGL(ffn_gate_up_bf16_kernel, dim3(g1), dim3(G::NT), lds, st, p.d, p.I, p.n_experts, p.n_rows,
                     p.a_rows, p.offsets, p.mode, p.row_src, static_cast<const uint16_t*>(p.a),
                     static_cast<const uint16_t*>(p.w_gu), static_cast<uint16_t*>(p.h));
  return hipGetLastError();
}

hipError_t launch_ffn_bf16_down(const FfnArgs& p, hipStream_t st) {
  using G = FfnTile;
  set_lds_limits();
  const size_t lds = G::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / G::BM + p.n_experts;
  const int g2 = persistent_grid(mblocks * (p.d / G::BN), 2);
  hipLaunchKernelGGL(ffn_down_bf16_kernel, dim3(g2), dim3(G::NT), lds, st, p.d, p.I, p.n_experts, p.n_rows,
                     p.offsets, static_cast<const uint16_t*>(p.h), static_cast<const uint16_t*>(p.w_d),
                     static_cast<uint16_t*>(p.y));
  return hipGetLastError();
}

}  // namespace moe
