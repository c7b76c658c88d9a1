// Grouped SwiGLU expert FFN in bf16 with fp32 MFMA accumulation
// ("DeepSeek_V3_Report: Annotation", SwiGLU paragraph and eq. (12)).
//
// Two persistent launches over all experts, one 512-thread workgroup (eight
// waves, two per SIMD) per CU, 256 weight rows x 320 token rows per tile on
// the pipelined direct-to-LDS main loop (gemm_w8.h) and balanced blocks (an
// expert's rows split into near-equal blocks of at most 320 rows, so an
// expert of the V3 shape streams its weights once; empty 32-row sub-tiles are
// skipped):
//  1. gate/up: H[r, c] = SiLU(x_r . Wg[c]) * (x_r . Wu[c]) for 128 H columns;
//     each wave holds 32 gate rows and the matching 32 up rows, so the SwiGLU
//     product is formed in registers. Token rows are read through the row
//     mode (the gather is fused into the operand load).
//  2. down:    y[r, n] = H_r . Wd[n] for 256 output columns.
// H lives in the workspace as bf16 [n_rows, I]. The weights come row-major
// (MOE_BF16) or in the tiled layout of moe_tile_weights_bf16 (MOE_BF16_TILED:
// every stage's weight loads read one contiguous 16 KB block).
#include <mutex>

#include "common.h"
#include "gemm_w8.h"
#include "launch.h"
#include "sched.h"

namespace moe {

using FP = W8<false>;              // 256 weight rows x 320 token rows per tile, eight waves
using FPT = W8<true>;              // the same with the weights in the tiled layout
constexpr int kHcols = FP::BW / 2;  // H columns per gate/up tile
constexpr int kMaxExpertsBf16 = 2048;   // the schedule's per-expert table shares the LDS with the ring

__device__ __forceinline__ void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// One gate/up tile: wave quarter ww holds the gate rows of H columns 32 ww .. 32 ww + 31 of the tile
// (tile rows 128 (ww >> 1) + 32 (ww & 1) ..) and the matching up rows (64 tile rows further), so the
// SwiGLU product forms in registers.
template <class P, int MS, int LT>
__device__ __forceinline__ void gate_up_tile(const W8Rows& rows, int d, int I, const Unit& un, uint8_t* lds,
                                             uint16_t* __restrict__ H, uint16_t* __restrict__ GU) {
  f32x16 acc[2][5];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  const int ww = wave_uniform((w8_tid() >> 6) & 3);
  const int wr0 = 128 * (ww >> 1) + 32 * (ww & 1);
  const W8Offs o = w8_offsets(wr0, wr0 + 64);
  w8_mainloop<P, MS, LT>(rows, d, lds, o, acc);
  const int tid = w8_tid(), h = (tid & 63) >> 5;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int tr = w8_token_row(i, tid);
    if (tr < un.rows) {
      const int c0 = un.nb * kHcols + ww * 32 + 4 * h;
      uint16_t* hrow = H + static_cast<size_t>(un.m0 + tr) * I + c0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_bf16x4(hrow + 8 * q, silu(acc[0][i][4 * q]) * acc[1][i][4 * q],
                     silu(acc[0][i][4 * q + 1]) * acc[1][i][4 * q + 1],
                     silu(acc[0][i][4 * q + 2]) * acc[1][i][4 * q + 2],
                     silu(acc[0][i][4 * q + 3]) * acc[1][i][4 * q + 3]);
      if (GU) {                                       // the SwiGLU inputs for the backward: [G | U] rows of 2I
        uint16_t* grow = GU + static_cast<size_t>(un.m0 + tr) * 2 * I + c0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          store_bf16x4(grow + 8 * q, acc[0][i][4 * q], acc[0][i][4 * q + 1], acc[0][i][4 * q + 2],
                       acc[0][i][4 * q + 3]);
          store_bf16x4(grow + I + 8 * q, acc[1][i][4 * q], acc[1][i][4 * q + 1], acc[1][i][4 * q + 2],
                       acc[1][i][4 * q + 3]);
        }
      }
    }
  }
}

// One down tile: wave quarter ww holds output columns 64 ww .. 64 ww + 63 of the tile.
template <class P, int MS, int LT>
__device__ __forceinline__ void down_tile(const W8Rows& rows, int d, int I, const Unit& un, uint8_t* lds,
                                          uint16_t* __restrict__ y) {
  f32x16 acc[2][5];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  const int ww = wave_uniform((w8_tid() >> 6) & 3);
  const W8Offs o = w8_offsets(64 * ww, 64 * ww + 32);
  w8_mainloop<P, MS, LT>(rows, I, lds, o, acc);
  const int tid = w8_tid(), h = (tid & 63) >> 5;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int tr = w8_token_row(i, tid);
    if (tr < un.rows) {
      uint16_t* yrow = y + static_cast<size_t>(un.m0 + tr) * d;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = un.nb * FP::BW + 64 * ww + 32 * j + 8 * q + 4 * h;
          if (col < d)                                // d % 256 == 128: the last tile has 128 columns
            store_bf16x4(yrow + col, acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                         acc[j][i][4 * q + 3]);
        }
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
  const int total = build_units_balanced(off, E, n_rows, FP::MAXSUB, NB, cum, wtmp);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced(t, off, E, n_rows, FP::MAXSUB, cum);
    int s_first = source_row(mode, row_src, un.m0, un.seg0, a_rows);
    if (s_first < 0) s_first = 0;
    W8Rows rows;
    rows.trs = pipe_rsrc(a, static_cast<uint64_t>(a_rows) * d * 2);
    const int tid = w8_tid();
#pragma unroll
    for (int q = 0; q < FP::TLMAX; ++q) {
      const int u = w8_unit(q, tid), r = w8_load_row(u, tid);
      int sr = r < un.rows ? source_row(mode, row_src, un.m0 + r, un.seg0, a_rows) : -1;
      if (sr < 0) sr = s_first;                       // rows past the block: any valid row, never stored
      rows.ot[q] = (static_cast<uint32_t>(sr) * d + w8_load_chunk(u, tid) * 8) * 2;
    }
    if (P::TILED) {                                   // tile nb: the gate and up rows of H columns 128 nb ..
      rows.wrs = pipe_rsrc(wgu + (static_cast<size_t>(un.e) * NB + un.nb) * FP::BW * d,
                           static_cast<uint64_t>(FP::BW) * d * 2);
    } else {
      rows.wrs = pipe_rsrc(wgu + static_cast<size_t>(un.e) * 2 * I * d, static_cast<uint64_t>(2 * I) * d * 2);
#pragma unroll
      for (int q = 0; q < FP::WL; ++q) {
        const int u = w8_unit(q, tid), rw = w8_load_row(u, tid);
        const int j = (rw >> 5) & 3;                  // sub-tiles 0,1 of each 128: gate rows; 2,3: the matching up rows
        const int hcol = un.nb * kHcols + (rw >> 7) * 64 + (j & 1) * 32 + (rw & 31);
        rows.ow[q] = (static_cast<uint32_t>(j >= 2 ? I + hcol : hcol) * d + w8_load_chunk(u, tid) * 8) * 2;
      }
    }
#define GU_CALL(MS, LT) gate_up_tile<P, MS, LT>(rows, d, I, un, lds_p, H, GU)
    W8_DISPATCH(un.nsub, GU_CALL);
#undef GU_CALL
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
  const int total = build_units_balanced(off, E, n_rows, FP::MAXSUB, NB, cum, wtmp);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced(t, off, E, n_rows, FP::MAXSUB, cum);
    W8Rows rows;
    rows.trs = pipe_rsrc(H, static_cast<uint64_t>(n_rows) * I * 2);
    const int tid = w8_tid();
#pragma unroll
    for (int q = 0; q < FP::TLMAX; ++q) {
      const int u = w8_unit(q, tid), r = w8_load_row(u, tid);
      rows.ot[q] = (static_cast<uint32_t>(un.m0 + (r < un.rows ? r : 0)) * I + w8_load_chunk(u, tid) * 8) * 2;
    }
    if (P::TILED) {                                   // ceil(d / 256) tiles per expert, the last padded with zeros
      rows.wrs = pipe_rsrc(wd + (static_cast<size_t>(un.e) * NB + un.nb) * FP::BW * I,
                           static_cast<uint64_t>(FP::BW) * I * 2);
    } else {
      rows.wrs = pipe_rsrc(wd + static_cast<size_t>(un.e) * d * I, static_cast<uint64_t>(d) * I * 2);
#pragma unroll
      for (int q = 0; q < FP::WL; ++q) {
        const int u = w8_unit(q, tid);
        rows.ow[q] =
            (static_cast<uint32_t>(min(un.nb * FP::BW + w8_load_row(u, tid), d - 1)) * I + w8_load_chunk(u, tid) * 8) * 2;
      }
    }
#define DN_CALL(MS, LT) down_tile<P, MS, LT>(rows, d, I, un, lds_p, y)
    W8_DISPATCH(un.nsub, DN_CALL);
#undef DN_CALL
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
    // ring + schedule for up to kMaxExpertsBf16 experts; a refused request must not leave a sticky error
    const int need = FP::LDS_BYTES + 4 * (kMaxExpertsBf16 + 1);
    static_assert(FP::LDS_BYTES + 4 * (kMaxExpertsBf16 + 1) + 128 <= 160 * 1024, "LDS budget");
    for (const void* k : {reinterpret_cast<const void*>(ffn_gate_up_bf16_kernel<FP>),
                          reinterpret_cast<const void*>(ffn_gate_up_bf16_kernel<FPT>),
                          reinterpret_cast<const void*>(ffn_down_bf16_kernel<FP>),
                          reinterpret_cast<const void*>(ffn_down_bf16_kernel<FPT>)})
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, need);
    (void)hipGetLastError();
  });
}

hipError_t launch_ffn_bf16_gate_up(const FfnArgs& p, hipStream_t st, bool tiled) {
  if (p.n_experts > kMaxExpertsBf16) return hipErrorInvalidValue;
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
  if (p.n_experts > kMaxExpertsBf16) return hipErrorInvalidValue;
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
