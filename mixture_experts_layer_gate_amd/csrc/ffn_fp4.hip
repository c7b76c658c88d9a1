// Grouped SwiGLU expert FFN with MXFP4 expert weights and E4M3 activations
// ("DeepSeek V3 / V4 Infra", V4 post-training FP4 QAT of the MoE expert
// weights; activations and H as in the V3 fp8 recipe of
// "DeepSeek_V3_Report: Annotation", section "Fine-Grained Quantization").
//
// Weights: E2M1 codes with one E8M0 scale per 32 consecutive K values, in the
// tiled layout of moe_quantize_weights_mxfp4 (per expert: ntiles tiles of 256
// rows, each K/64 code blocks of 8 KB and K/128 scale blocks of 1 KB; the
// gate/up tile t holds the gate and up rows of H columns 128 t .. 128 t + 127
// in the order the tile's waves use them); the MFMA applies the scales itself
// (gemm_pipe4.h). The schedule,
// the unit queue and the epilogues are those of the E4M3-weight kernels:
//  1. gate/up: H = SiLU(g) * u, re-quantised per 1x128 tile along I (E4M3 codes
//     and fp32 scales);
//  2. down: y = H . Wd, bf16 out.
#include <mutex>

#include "common.h"
#include "ffn_epi8.h"
#include "gemm_pipe4.h"
#include "launch.h"
#include "sched.h"

namespace moe {

using P4 = Pipe4;
constexpr int kMaxExperts4 = 2048;   // the schedule's per-expert table shares the LDS with the ring

template <int MS, int LT>
__device__ __forceinline__ void gate_up4_unit(const Pipe4Rows& rows, __amdgpu_buffer_rsrc_t tsrs, int d, int I,
                                              const Unit& un, int nb0, int nseg, uint8_t* lds,
                                              uint8_t* __restrict__ Hq, float* __restrict__ Hs) {
  GateUpEpi8<MS, P4::AMAX_OFF> epi{un, I, nb0, lds, Hq, Hs};
  pipe4_stream<MS, LT>(rows, tsrs, d, nseg, lds, epi);
}

template <int MS, int LT>
__device__ __forceinline__ void down4_unit(const Pipe4Rows& rows, __amdgpu_buffer_rsrc_t tsrs, int d, int I,
                                           const Unit& un, int nb0, int nseg, uint8_t* lds, uint16_t* __restrict__ y) {
  DownEpi8<MS> epi{un, d, nb0, y};
  pipe4_stream<MS, LT>(rows, tsrs, I, nseg, lds, epi);
}

// The weight codes and scales of expert e from tile t0 on, nseg tiles of a
// matrix with K columns and ntiles tiles.
__device__ __forceinline__ void pipe4_weights(Pipe4Rows& rows, const uint8_t* codes, const uint8_t* scales, int e,
                                              int ntiles, int t0, int nseg, int K) {
  const size_t tile = static_cast<size_t>(e) * ntiles + t0;
  rows.wrs = pipe_rsrc(codes + tile * P4::BW * (K / 2), static_cast<uint64_t>(nseg) * P4::BW * (K / 2));
  rows.srs = pipe_rsrc(scales + tile * P4::BW * (K / 32), static_cast<uint64_t>(nseg) * P4::BW * (K / 32));
}

__global__ __launch_bounds__(P4::NT, 1) void ffn_gate_up_fp4_kernel(
    int d, int I, int E, int n_rows, int a_rows, const int32_t* __restrict__ off, moe_row_mode mode,
    const int32_t* __restrict__ row_src, const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ wgu, const uint8_t* __restrict__ wgu_scale, uint8_t* __restrict__ Hq,
    float* __restrict__ Hs, int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t lds4[];
  int* srcrow = reinterpret_cast<int*>(lds4 + P4::SRC_OFF);
  int* cum = reinterpret_cast<int*>(lds4 + P4::LDS_BYTES);
  __shared__ int wtmp[16];
  const int kc = d / 128, NB = I / 128;
  const int total = build_units_balanced(off, E, n_rows, kMaxSub8, cdiv(NB, P4::MAX_SEG), cum, wtmp);
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t trs = pipe_rsrc(a, static_cast<uint64_t>(a_rows) * d);
  const __amdgpu_buffer_rsrc_t tsrs = pipe_rsrc(a_scale, static_cast<uint64_t>(a_rows) * kc * 4);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced<false>(t, off, E, n_rows, kMaxSub8, cum);
    const int nb0 = un.nb * P4::MAX_SEG, nseg = min(P4::MAX_SEG, NB - nb0);
    if (tid < P4::BT) {
      int s_first = source_row(mode, row_src, un.m0, un.seg0, a_rows);
      if (s_first < 0) s_first = 0;
      const int sr = tid < un.rows ? source_row(mode, row_src, un.m0 + tid, un.seg0, a_rows) : -1;
      srcrow[tid] = sr < 0 ? s_first : sr;
    }
    __syncthreads();
    Pipe4Rows rows;
    rows.trs = trs;
#pragma unroll
    for (int q = 0; q < P4::TL; ++q)
      rows.ot[q] = static_cast<uint32_t>(srcrow[pipe8_load_row(q)]) * d + pipe8_load_chunk(q) * 16;
    pipe4_weights(rows, wgu, wgu_scale, un.e, NB, nb0, nseg, d);
    const bool full = live_token_subtiles8(un.nsub) * 2 >= un.nsub;
    if (un.nsub > 2) {
      if (full) gate_up4_unit<2, 2>(rows, tsrs, d, I, un, nb0, nseg, lds4, Hq, Hs);
      else gate_up4_unit<1, 2>(rows, tsrs, d, I, un, nb0, nseg, lds4, Hq, Hs);
    } else {
      if (full) gate_up4_unit<1, 1>(rows, tsrs, d, I, un, nb0, nseg, lds4, Hq, Hs);
      else gate_up4_unit<0, 1>(rows, tsrs, d, I, un, nb0, nseg, lds4, Hq, Hs);
    }
  }
}

__global__ __launch_bounds__(P4::NT, 1) void ffn_down_fp4_kernel(int d, int I, int E, int n_rows,
                                                                 const int32_t* __restrict__ off,
                                                                 const uint8_t* __restrict__ Hq,
                                                                 const float* __restrict__ Hs,
                                                                 const uint8_t* __restrict__ wd,
                                                                 const uint8_t* __restrict__ wd_scale,
                                                                 uint16_t* __restrict__ y, int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t lds4[];
  int* srcrow = reinterpret_cast<int*>(lds4 + P4::SRC_OFF);
  int* cum = reinterpret_cast<int*>(lds4 + P4::LDS_BYTES);
  __shared__ int wtmp[16];
  // Output-column tiles of 256 in groups of MAX_SEG per unit; when d % 256 == 128
  // the last 128 columns form a group of their own: the layout pads their tile
  // to 256 rows (zero codes) and their outputs past d are never stored.
  const int kc = I / 128, NBF = d / P4::BW, NGF = cdiv(NBF, P4::MAX_SEG);
  const int NG = NGF + (d % P4::BW ? 1 : 0), NG4 = cdiv(d, P4::BW);
  const int total = build_units_balanced(off, E, n_rows, kMaxSub8, NG, cum, wtmp);
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t trs = pipe_rsrc(Hq, static_cast<uint64_t>(n_rows) * I);
  const __amdgpu_buffer_rsrc_t tsrs = pipe_rsrc(Hs, static_cast<uint64_t>(n_rows) * kc * 4);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced<false>(t, off, E, n_rows, kMaxSub8, cum);
    const int nb0 = un.nb < NGF ? un.nb * P4::MAX_SEG : NBF;
    const int nseg = un.nb < NGF ? min(P4::MAX_SEG, NBF - nb0) : 1;
    if (tid < P4::BT) srcrow[tid] = un.m0 + (tid < un.rows ? tid : 0);
    __syncthreads();
    Pipe4Rows rows;
    rows.trs = trs;
#pragma unroll
    for (int q = 0; q < P4::TL; ++q)
      rows.ot[q] = static_cast<uint32_t>(srcrow[pipe8_load_row(q)]) * I + pipe8_load_chunk(q) * 16;
    pipe4_weights(rows, wd, wd_scale, un.e, NG4, nb0, nseg, I);
    const bool full = live_token_subtiles8(un.nsub) * 2 >= un.nsub;
    if (un.nsub > 2) {
      if (full) down4_unit<2, 2>(rows, tsrs, d, I, un, nb0, nseg, lds4, y);
      else down4_unit<1, 2>(rows, tsrs, d, I, un, nb0, nseg, lds4, y);
    } else {
      if (full) down4_unit<1, 1>(rows, tsrs, d, I, un, nb0, nseg, lds4, y);
      else down4_unit<0, 1>(rows, tsrs, d, I, un, nb0, nseg, lds4, y);
    }
  }
}

static int f4_grid(long long units_upper) {
  long long g = static_cast<long long>(device_cu_count());   // one workgroup per CU
  if (units_upper < g) g = units_upper;
  g = ((g + 7) / 8) * 8;
  return static_cast<int>(g < 8 ? 8 : g);
}

static void f4_set_lds_limits() {
  static std::once_flag once;
  std::call_once(once, [] {
    const int need = P4::LDS_BYTES + 4 * (kMaxExperts4 + 1);
    static_assert(P4::LDS_BYTES + 4 * (kMaxExperts4 + 1) + 64 <= 160 * 1024, "LDS budget");
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_gate_up_fp4_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, need);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_down_fp4_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, need);
    (void)hipGetLastError();
  });
}

hipError_t launch_ffn_fp4_gate_up(const FfnArgs& p, hipStream_t st) {
  if (p.n_experts > kMaxExperts4) return hipErrorInvalidValue;
  f4_set_lds_limits();
  int* q = p.queue;
  if (hipError_t e = launch_queue_reset(q, st); e != hipSuccess) return e;
  const size_t lds = P4::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / P4::BT + p.n_experts;
  hipLaunchKernelGGL(ffn_gate_up_fp4_kernel, dim3(f4_grid(mblocks * cdiv(p.I / 128, P4::MAX_SEG))), dim3(P4::NT), lds,
                     st, p.d, p.I, p.n_experts, p.n_rows, p.a_rows, p.offsets, p.mode, p.row_src,
                     static_cast<const uint8_t*>(p.a), p.a_scale, static_cast<const uint8_t*>(p.w_gu),
                     static_cast<const uint8_t*>(p.w_gu_scale), static_cast<uint8_t*>(p.h), p.h_scale, q);
  return hipGetLastError();
}

hipError_t launch_ffn_fp4_down(const FfnArgs& p, hipStream_t st) {
  if (p.n_experts > kMaxExperts4) return hipErrorInvalidValue;
  f4_set_lds_limits();
  int* q = p.queue;
  if (hipError_t e = launch_queue_reset(q, st); e != hipSuccess) return e;
  const size_t lds = P4::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / P4::BT + p.n_experts;
  hipLaunchKernelGGL(ffn_down_fp4_kernel, dim3(f4_grid(mblocks * (cdiv(p.d / P4::BW, P4::MAX_SEG) + 1))),
                     dim3(P4::NT), lds, st, p.d, p.I, p.n_experts, p.n_rows, p.offsets,
                     static_cast<const uint8_t*>(p.h), p.h_scale, static_cast<const uint8_t*>(p.w_d),
                     static_cast<const uint8_t*>(p.w_d_scale), static_cast<uint16_t*>(p.y), q);
  return hipGetLastError();
}

}  // namespace moe
