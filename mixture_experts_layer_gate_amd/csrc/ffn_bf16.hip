// Grouped SwiGLU expert FFN in bf16 with fp32 MFMA accumulation
// ("DeepSeek_V3_Report: Annotation", SwiGLU paragraph and eq. (12)).
//
// Two persistent launches over all experts, one 256-thread workgroup per CU,
// 256 weight rows x 256 token rows per tile on the pipelined direct-to-LDS
// main loop (gemm_pipe.h) and balanced blocks (an expert's rows split into
// near-equal blocks of at most 256 rows; empty 32-row sub-tiles are skipped):
//  1. gate/up: H[r, c] = SiLU(x_r . Wg[c]) * (x_r . Wu[c]) for 128 H columns;
//     each wave holds 64 gate rows and the matching 64 up rows, so the SwiGLU
//     product is formed in registers. Token rows are read through the row
//     mode (the gather is fused into the operand load).
//  2. down:    y[r, n] = H_r . Wd[n] for 256 output columns.
// H lives in the workspace as bf16 [n_rows, I]. The weights come row-major
// (MOE_BF16) or in the tiled layout of moe_tile_weights_bf16 (MOE_BF16_TILED:
// every stage's weight loads read one contiguous 16 KB block).
#include <mutex>

#include "common.h"
#include "gemm_pipe.h"
#include "launch.h"
#include "sched.h"

namespace moe {

using FP = Pipe<256, 256>;         // 256 weight rows x 256 token rows per tile, waves of 128 x 128
using FPT = Pipe<256, 256, true>;  // the same with the weights in the tiled layout
constexpr int kHcols = FP::BW / 2;  // H columns per gate/up tile

__device__ __forceinline__ int live_token_subtiles(int nsub) {
  const int wt = (threadIdx.x >> 6) & 1;
  return clampi((nsub - wt + 1) / 2, 0, 4);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// One tile with MS live token sub-tiles per wave and LT token load groups per
// stage: main loop and epilogue in one instantiation, so the accumulators
// never merge across variants.
template <class P, int MS, int LT>
__device__ __forceinline__ void gate_up_tile(const PipeRows<P>& rows, int d, int I, const Unit& un, uint8_t* lds,
                                             uint16_t* __restrict__ H, uint16_t* __restrict__ GU) {
  f32x16 acc[FP::TW][FP::TT];
#pragma unroll
  for (int j = 0; j < FP::TW; ++j)
#pragma unroll
    for (int i = 0; i < FP::TT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  pipe_mainloop<P, MS, LT>(rows, d, lds, acc);
  const int ww = threadIdx.x >> 7, h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int tr = pipe_token_row(i);
    if (tr < un.rows) {
      uint16_t* hrow = H + static_cast<size_t>(un.m0 + tr) * I + un.nb * kHcols + ww * 64 + 4 * h;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          store_bf16x4(hrow + j * 32 + 8 * q, silu(acc[j][i][4 * q]) * acc[j + 2][i][4 * q],
                       silu(acc[j][i][4 * q + 1]) * acc[j + 2][i][4 * q + 1],
                       silu(acc[j][i][4 * q + 2]) * acc[j + 2][i][4 * q + 2],
                       silu(acc[j][i][4 * q + 3]) * acc[j + 2][i][4 * q + 3]);
      if (GU) {                                       // the SwiGLU inputs for the backward: [G | U] rows of 2I
        uint16_t* grow = GU + static_cast<size_t>(un.m0 + tr) * 2 * I + un.nb * kHcols + ww * 64 + 4 * h;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            store_bf16x4(grow + j * 32 + 8 * q, acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                         acc[j][i][4 * q + 3]);
            store_bf16x4(grow + I + j * 32 + 8 * q, acc[j + 2][i][4 * q], acc[j + 2][i][4 * q + 1],
                         acc[j + 2][i][4 * q + 2], acc[j + 2][i][4 * q + 3]);
          }
      }
    }
  }
}

template <class P, int MS, int LT>
__device__ __forceinline__ void down_tile(const PipeRows<P>& rows, int d, int I, const Unit& un, uint8_t* lds,
                                          uint16_t* __restrict__ y) {
  f32x16 acc[FP::TW][FP::TT];
#pragma unroll
  for (int j = 0; j < FP::TW; ++j)
#pragma unroll
    for (int i = 0; i < FP::TT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  pipe_mainloop<P, MS, LT>(rows, I, lds, acc);
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int tr = pipe_token_row(i);
    if (tr < un.rows) {
      uint16_t* yrow = y + static_cast<size_t>(un.m0 + tr) * d + un.nb * FP::BW;
#pragma unroll
      for (int j = 0; j < FP::TW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (un.nb * FP::BW + pipe_wcol<FP>(j, q) < d)   // d % 256 == 128: the last tile has 128 columns
            store_bf16x4(yrow + pipe_wcol<FP>(j, q), acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                         acc[j][i][4 * q + 3]);
    }
  }
}

template <class P>
__global__ __launch_bounds__(FP::NT, 1) void ffn_gate_up_bf16_kernel(
    int d, int I, int E, int n_rows, int a_rows, const int32_t* __restrict__ off, moe_row_mode mode,
    const int32_t* __restrict__ row_src, const uint16_t* __restrict__ a, const uint16_t* __restrict__ wgu,
    uint16_t* __restrict__ H, uint16_t* __restrict__ GU, int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t lds_p[];
  int* cum = reinterpret_cast<int*>(lds_p + FP::LDS_BYTES);
  __shared__ int wtmp[16];
  const int NB = I / kHcols;
  const int total = build_units_balanced(off, E, n_rows, FP::BT / 32, NB, cum, wtmp);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced(t, off, E, n_rows, FP::BT / 32, cum);
    int s_first = source_row(mode, row_src, un.m0, un.seg0, a_rows);
    if (s_first < 0) s_first = 0;
    PipeRows<P> rows;
    rows.trs = pipe_rsrc(a, static_cast<uint64_t>(a_rows) * d * 2);
#pragma unroll
    for (int q = 0; q < FP::TL; ++q) {
      const int r = pipe_load_row(q);
      int sr = r < un.rows ? source_row(mode, row_src, un.m0 + r, un.seg0, a_rows) : -1;
      if (sr < 0) sr = s_first;                       // rows past the block: any valid row, never stored
      rows.ot[q] = (static_cast<uint32_t>(sr) * d + pipe_load_chunk(q) * 8) * 2;
    }
    if (P::TILED) {                                   // tile nb: the gate and up rows of H columns 128 nb ..
      rows.wrs = pipe_rsrc(wgu + (static_cast<size_t>(un.e) * NB + un.nb) * FP::BW * d,
                           static_cast<uint64_t>(FP::BW) * d * 2);
#pragma unroll
      for (int q = 0; q < FP::WL; ++q) rows.ow[q] = ((q * 4 + (threadIdx.x >> 6)) * 64 + (threadIdx.x & 63)) * 16;
    } else {
      rows.wrs = pipe_rsrc(wgu + static_cast<size_t>(un.e) * 2 * I * d, static_cast<uint64_t>(2 * I) * d * 2);
#pragma unroll
      for (int q = 0; q < FP::WL; ++q) {
        const int rw = pipe_load_row(q);
        const int j = (rw >> 5) & 3;                  // sub-tiles 0,1: gate rows; 2,3: the matching up rows
        const int hcol = un.nb * kHcols + (rw >> 7) * 64 + (j & 1) * 32 + (rw & 31);
        rows.ow[q] = (static_cast<uint32_t>(j >= 2 ? I + hcol : hcol) * d + pipe_load_chunk(q) * 8) * 2;
      }
    }
    // LT = ceil(nsub / 2) token load groups; wave row 0 has LT live sub-tiles, row 1 LT or LT - 1
    const bool full = live_token_subtiles(un.nsub) * 2 >= un.nsub;
    switch ((un.nsub + 1) / 2) {
      case 4: full ? gate_up_tile<P, 4, 4>(rows, d, I, un, lds_p, H, GU) : gate_up_tile<P, 3, 4>(rows, d, I, un, lds_p, H, GU); break;
      case 3: full ? gate_up_tile<P, 3, 3>(rows, d, I, un, lds_p, H, GU) : gate_up_tile<P, 2, 3>(rows, d, I, un, lds_p, H, GU); break;
      case 2: full ? gate_up_tile<P, 2, 2>(rows, d, I, un, lds_p, H, GU) : gate_up_tile<P, 1, 2>(rows, d, I, un, lds_p, H, GU); break;
      default: full ? gate_up_tile<P, 1, 1>(rows, d, I, un, lds_p, H, GU) : gate_up_tile<P, 0, 1>(rows, d, I, un, lds_p, H, GU); break;
    }
  }
}

template <class P>
__global__ __launch_bounds__(FP::NT, 1) void ffn_down_bf16_kernel(int d, int I, int E, int n_rows,
                                                                  const int32_t* __restrict__ off,
                                                                  const uint16_t* __restrict__ H,
                                                                  const uint16_t* __restrict__ wd,
                                                                  uint16_t* __restrict__ y,
                                                                  int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t lds_p[];
  int* cum = reinterpret_cast<int*>(lds_p + FP::LDS_BYTES);
  __shared__ int wtmp[16];
  const int NB = cdiv(d, FP::BW);                    // the last tile has 128 columns when d % 256 == 128
  const int total = build_units_balanced(off, E, n_rows, FP::BT / 32, NB, cum, wtmp);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced(t, off, E, n_rows, FP::BT / 32, cum);
    PipeRows<P> rows;
    rows.trs = pipe_rsrc(H, static_cast<uint64_t>(n_rows) * I * 2);
#pragma unroll
    for (int q = 0; q < FP::TL; ++q) {
      const int r = pipe_load_row(q);
      rows.ot[q] = (static_cast<uint32_t>(un.m0 + (r < un.rows ? r : 0)) * I + pipe_load_chunk(q) * 8) * 2;
    }
    if (P::TILED) {                                   // ceil(d / 256) tiles per expert, the last padded with zeros
      rows.wrs = pipe_rsrc(wd + (static_cast<size_t>(un.e) * NB + un.nb) * FP::BW * I,
                           static_cast<uint64_t>(FP::BW) * I * 2);
#pragma unroll
      for (int q = 0; q < FP::WL; ++q) rows.ow[q] = ((q * 4 + (threadIdx.x >> 6)) * 64 + (threadIdx.x & 63)) * 16;
    } else {
      rows.wrs = pipe_rsrc(wd + static_cast<size_t>(un.e) * d * I, static_cast<uint64_t>(d) * I * 2);
#pragma unroll
      for (int q = 0; q < FP::WL; ++q)
        rows.ow[q] =
            (static_cast<uint32_t>(min(un.nb * FP::BW + pipe_load_row(q), d - 1)) * I + pipe_load_chunk(q) * 8) * 2;
    }
    const bool full = live_token_subtiles(un.nsub) * 2 >= un.nsub;
    switch ((un.nsub + 1) / 2) {
      case 4: full ? down_tile<P, 4, 4>(rows, d, I, un, lds_p, y) : down_tile<P, 3, 4>(rows, d, I, un, lds_p, y); break;
      case 3: full ? down_tile<P, 3, 3>(rows, d, I, un, lds_p, y) : down_tile<P, 2, 3>(rows, d, I, un, lds_p, y); break;
      case 2: full ? down_tile<P, 2, 2>(rows, d, I, un, lds_p, y) : down_tile<P, 1, 2>(rows, d, I, un, lds_p, y); break;
      default: full ? down_tile<P, 1, 1>(rows, d, I, un, lds_p, y) : down_tile<P, 0, 1>(rows, d, I, un, lds_p, y); break;
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
    // ring + schedule for up to 4096 experts; a refused request must not leave a sticky error
    const int need = FP::LDS_BYTES + 4 * 4097;
    for (const void* k : {reinterpret_cast<const void*>(ffn_gate_up_bf16_kernel<FP>),
                          reinterpret_cast<const void*>(ffn_gate_up_bf16_kernel<FPT>),
                          reinterpret_cast<const void*>(ffn_down_bf16_kernel<FP>),
                          reinterpret_cast<const void*>(ffn_down_bf16_kernel<FPT>)})
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, need);
    (void)hipGetLastError();
  });
}

hipError_t launch_ffn_bf16_gate_up(const FfnArgs& p, hipStream_t st, bool tiled) {
  set_lds_limits();
  int* q = p.queue;
  if (hipError_t e = launch_queue_reset(q, st); e != hipSuccess) return e;
  const size_t lds = FP::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / FP::BT + p.n_experts;
  const int g1 = persistent_grid(mblocks * (p.I / kHcols), 1);
  hipLaunchKernelGGL(tiled ? ffn_gate_up_bf16_kernel<FPT> : ffn_gate_up_bf16_kernel<FP>, dim3(g1), dim3(FP::NT), lds,
                     st, p.d, p.I, p.n_experts, p.n_rows,
                     p.a_rows, p.offsets, p.mode, p.row_src, static_cast<const uint16_t*>(p.a),
                     static_cast<const uint16_t*>(p.w_gu), static_cast<uint16_t*>(p.h),
                     static_cast<uint16_t*>(p.gu_cache), q);
  return hipGetLastError();
}

hipError_t launch_ffn_bf16_down(const FfnArgs& p, hipStream_t st, bool tiled) {
  set_lds_limits();
  int* q = p.queue;
  if (hipError_t e = launch_queue_reset(q, st); e != hipSuccess) return e;
  const size_t lds = FP::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / FP::BT + p.n_experts;
  const int g2 = persistent_grid(mblocks * cdiv(p.d, FP::BW), 1);
  hipLaunchKernelGGL(tiled ? ffn_down_bf16_kernel<FPT> : ffn_down_bf16_kernel<FP>, dim3(g2), dim3(FP::NT), lds, st,
                     p.d, p.I, p.n_experts, p.n_rows,
                     p.offsets, static_cast<const uint16_t*>(p.h), static_cast<const uint16_t*>(p.w_d),
                     static_cast<uint16_t*>(p.y), q);
  return hipGetLastError();
}

}  // namespace moe
