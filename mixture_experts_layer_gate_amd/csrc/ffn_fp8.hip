// Grouped SwiGLU expert FFN with E4M3 operands ("DeepSeek_V3_Report: Annotation",
// sections "Fine-Grained Quantization" and "Increasing Accumulation Precision";
// "DeepSeek V3 / V4 Infra", V3 FP8 section).
//
// Activations carry one fp32 scale per 1x128 tile (row, K chunk), weights one
// per 128x128 block; every 128-wide K chunk of the products is scaled by the
// product of the two scales in fp32 (gemm_pipe8.h, gemm_f8w.h). The weight
// codes come in the tiled layout of moe_quantize_weights (per expert, tiles of
// 256 rows whose 64-wide K steps are contiguous 16 KB blocks in LDS order).
// Two persistent launches over all experts, one workgroup per CU; a unit
// streams consecutive output-column tiles of one token block (up to two in the
// eight-wave gate/up, four otherwise). Two
// main loops:
//  * eight waves, 256 weight rows x 256 token rows per tile, an expert's rows
//    in near-equal blocks of at most eight 32-row sub-tiles (gemm_f8w.h):
//    K a multiple of 1024, whole 256-column output tiles, up to 1024 experts;
//    a 256-row expert streams its weights once;
//  * four waves, 256 x 128 tiles, blocks of four sub-tiles with the
//    remainder last (gemm_pipe8.h): every other shape.
//  1. gate/up: H[r, c] = SiLU(g) * u for 128 H columns per tile (each wave 64
//     gate rows + the matching 64 up rows, so the product forms in registers);
//     H is then re-quantised per 1x128 tile along I -- the tile owns exactly
//     one such tile per row: amax over its 128 columns, inv = fl32(448 / amax),
//     codes = E4M3(fl32(h * inv)), scale = fl32(amax / 448) (1 for amax = 0).
//  2. down: y[r, n] = H_r . Wd[n] for 256 output columns, bf16 out.
#include <mutex>

#include "common.h"
#include "ffn_epi8.h"
#include "gemm_f8w.h"
#include "gemm_pipe8.h"
#include "launch.h"
#include "sched.h"

namespace moe {

constexpr int kMaxExperts8 = 4096;

template <int MS, int LT>
__device__ __forceinline__ void gate_up8_unit(const Pipe8Rows& rows, __amdgpu_buffer_rsrc_t srs, int d, int I,
                                              const Unit& un, int nb0, int nseg, uint8_t* lds,
                                              uint8_t* __restrict__ Hq, float* __restrict__ Hs,
                                              uint8_t* __restrict__ GUq, float* __restrict__ GUs) {
  GateUpEpi8<MS, P8::AMAX_OFF> epi{un, I, nb0, lds, Hq, Hs, GUq, GUs};
  pipe8_stream<MS, LT, true>(rows, srs, d, nseg, lds, epi);
}

template <int MS, int LT>
__device__ __forceinline__ void down8_unit(const Pipe8Rows& rows, __amdgpu_buffer_rsrc_t srs, int d, int I,
                                           const Unit& un, int nb0, int nseg, uint8_t* lds,
                                           uint16_t* __restrict__ y, float* __restrict__ yf) {
  DownEpi8<MS> epi{un, d, nb0, y, yf};
  pipe8_stream<MS, LT, false>(rows, srs, I, nseg, lds, epi);
}

__global__ __launch_bounds__(P8::NT, 1) void ffn_gate_up_fp8_kernel(
    int d, int I, int E, int n_rows, int a_rows, const int32_t* __restrict__ off, moe_row_mode mode,
    const int32_t* __restrict__ row_src, const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ wgu, const float* __restrict__ wgu_scale, uint8_t* __restrict__ Hq,
    float* __restrict__ Hs, uint8_t* __restrict__ GUq, float* __restrict__ GUs, int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t lds8[];
  float* swt = reinterpret_cast<float*>(lds8 + P8::SW_OFF);
  int* srcrow = reinterpret_cast<int*>(lds8 + P8::SRC_OFF);
  int* cum = reinterpret_cast<int*>(lds8 + P8::LDS_BYTES);
  __shared__ int wtmp[16];
  const int kc = d / 128, NB = I / 128;
  const int total = build_units_balanced(off, E, n_rows, kMaxSub8, cdiv(NB, P8::MAX_SEG), cum, wtmp);
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t trs = pipe_rsrc(a, static_cast<uint64_t>(a_rows) * d);
  const __amdgpu_buffer_rsrc_t srs = pipe_rsrc(a_scale, static_cast<uint64_t>(a_rows) * kc * 4);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced<false>(t, off, E, n_rows, kMaxSub8, cum);
    const int nb0 = un.nb * P8::MAX_SEG, nseg = min(P8::MAX_SEG, NB - nb0);
    // LDS tables of the unit: weight scales of each tile (gate block row nb,
    // up block row I/128 + nb) and the source row of each tile row (rows past
    // the block read any valid row and are never stored)
    const float* sexp = wgu_scale + static_cast<size_t>(un.e) * (2 * I / 128) * kc;
    for (int x = tid; x < nseg * 2 * kc; x += P8::NT) {
      const int sb = x / kc, c = x - sb * kc, seg = sb >> 1, b = sb & 1;
      swt[(seg * 2 + b) * P8::MAX_CHUNKS + c] = sexp[static_cast<size_t>(b ? I / 128 + nb0 + seg : nb0 + seg) * kc + c];
    }
    if (tid < P8::BT) {
      int s_first = source_row(mode, row_src, un.m0, un.seg0, a_rows);
      if (s_first < 0) s_first = 0;
      const int sr = tid < un.rows ? source_row(mode, row_src, un.m0 + tid, un.seg0, a_rows) : -1;
      srcrow[tid] = sr < 0 ? s_first : sr;
    }
    __syncthreads();
    Pipe8Rows rows;
    rows.trs = trs;
#pragma unroll
    for (int q = 0; q < P8::TL; ++q)
      rows.ot[q] = static_cast<uint32_t>(srcrow[pipe8_load_row(q)]) * d + pipe8_load_chunk(q) * 16;
    // tiled weights: tile nb holds the gate and up rows of H columns 128 nb .. +127 (each wave half 64 of
    // them: sub-tiles 0, 1 the gate rows, 2, 3 the matching up rows), 256 rows x d bytes per tile
    rows.wrs = pipe_rsrc(wgu + (static_cast<size_t>(un.e) * NB + nb0) * P8::BW * d,
                         static_cast<uint64_t>(nseg) * P8::BW * d);
    // LT = ceil(nsub / 2) token load groups; wave row 0 has LT live sub-tiles, row 1 LT or LT - 1
    const bool full = live_token_subtiles8(un.nsub) * 2 >= un.nsub;
    if (un.nsub > 2) {
      if (full) gate_up8_unit<2, 2>(rows, srs, d, I, un, nb0, nseg, lds8, Hq, Hs, GUq, GUs);
      else gate_up8_unit<1, 2>(rows, srs, d, I, un, nb0, nseg, lds8, Hq, Hs, GUq, GUs);
    } else {
      if (full) gate_up8_unit<1, 1>(rows, srs, d, I, un, nb0, nseg, lds8, Hq, Hs, GUq, GUs);
      else gate_up8_unit<0, 1>(rows, srs, d, I, un, nb0, nseg, lds8, Hq, Hs, GUq, GUs);
    }
  }
}

__global__ __launch_bounds__(P8::NT, 1) void ffn_down_fp8_kernel(int d, int I, int E, int n_rows,
                                                                 const int32_t* __restrict__ off,
                                                                 const uint8_t* __restrict__ Hq,
                                                                 const float* __restrict__ Hs,
                                                                 const uint8_t* __restrict__ wd,
                                                                 const float* __restrict__ wd_scale,
                                                                 uint16_t* __restrict__ y, float* __restrict__ yf,
                                                                 int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t lds8[];
  float* swt = reinterpret_cast<float*>(lds8 + P8::SW_OFF);
  int* srcrow = reinterpret_cast<int*>(lds8 + P8::SRC_OFF);
  int* cum = reinterpret_cast<int*>(lds8 + P8::LDS_BYTES);
  __shared__ int wtmp[16];
  // Output-column tiles of 256 in groups of MAX_SEG per unit; when d % 256 == 128
  // the last 128 columns form a group of their own (their tile is padded with
  // zero codes; outputs past d are never stored).
  const int kc = I / 128, NBF = d / P8::BW, NGF = cdiv(NBF, P8::MAX_SEG);
  const int NG = NGF + (d % P8::BW ? 1 : 0), NG8 = cdiv(d, P8::BW);
  const int total = build_units_balanced(off, E, n_rows, kMaxSub8, NG, cum, wtmp);
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t trs = pipe_rsrc(Hq, static_cast<uint64_t>(n_rows) * I);
  const __amdgpu_buffer_rsrc_t srs = pipe_rsrc(Hs, static_cast<uint64_t>(n_rows) * kc * 4);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced<false>(t, off, E, n_rows, kMaxSub8, cum);
    const int nb0 = un.nb < NGF ? un.nb * P8::MAX_SEG : NBF;
    const int nseg = un.nb < NGF ? min(P8::MAX_SEG, NBF - nb0) : 1;
    // weight scales: wave half ww of tile nb covers output columns nb*256 + 128ww .. +127 = block row 2nb + ww
    // (past d: no block, factor 1, never stored)
    const float* sexp = wd_scale + static_cast<size_t>(un.e) * (d / 128) * kc;
    for (int x = tid; x < nseg * 2 * kc; x += P8::NT) {
      const int sb = x / kc, c = x - sb * kc, br = 2 * nb0 + sb;
      swt[sb * P8::MAX_CHUNKS + c] = br < d / 128 ? sexp[static_cast<size_t>(br) * kc + c] : 1.0f;
    }
    if (tid < P8::BT) srcrow[tid] = un.m0 + (tid < un.rows ? tid : 0);
    __syncthreads();
    Pipe8Rows rows;
    rows.trs = trs;
#pragma unroll
    for (int q = 0; q < P8::TL; ++q)
      rows.ot[q] = static_cast<uint32_t>(srcrow[pipe8_load_row(q)]) * I + pipe8_load_chunk(q) * 16;
    // tiled weights: ceil(d / 256) tiles of 256 output rows x I bytes per expert (the last padded with zero
    // codes when d % 256 == 128)
    rows.wrs = pipe_rsrc(wd + (static_cast<size_t>(un.e) * NG8 + nb0) * P8::BW * I,
                         static_cast<uint64_t>(nseg) * P8::BW * I);
    const bool full = live_token_subtiles8(un.nsub) * 2 >= un.nsub;
    if (un.nsub > 2) {
      if (full) down8_unit<2, 2>(rows, srs, d, I, un, nb0, nseg, lds8, y, yf);
      else down8_unit<1, 2>(rows, srs, d, I, un, nb0, nseg, lds8, y, yf);
    } else {
      if (full) down8_unit<1, 1>(rows, srs, d, I, un, nb0, nseg, lds8, y, yf);
      else down8_unit<0, 1>(rows, srs, d, I, un, nb0, nseg, lds8, y, yf);
    }
  }
}

// ---- eight-wave kernels (gemm_f8w.h) ----

constexpr int kMaxExpertsW = 1024;
// Output-column tiles per unit of the eight-wave gate/up (the down projection streams F8W::MAX_SEG): with 16
// tiles per token block at the V3 shape, units of two balance the CUs better than units of four (gate/up
// 3.02-3.06 -> 2.95-2.97 ms; the down projection, K = 2048, keeps four: 1.84 against 1.87 ms with two).
constexpr int kGateUpSegW = 2;
static_assert(kGateUpSegW <= F8W::MAX_SEG, "weight-scale table slots");

template <int MS, int LT>
__device__ __forceinline__ void gate_up8w_unit(const F8WRows& rows, int d, int I, const Unit& un, int nb0, int nseg,
                                               uint8_t* lds, uint8_t* __restrict__ Hq, float* __restrict__ Hs,
                                               uint8_t* __restrict__ GUq, float* __restrict__ GUs) {
  GateUpEpi8<MS, F8W::AMAX_OFF, F8WLayout> epi{un, I, nb0, lds, Hq, Hs, GUq, GUs};
  f8w_stream<MS, LT, true>(rows, d, nseg, lds, epi);
}

template <int MS, int LT>
__device__ __forceinline__ void down8w_unit(const F8WRows& rows, int d, int I, const Unit& un, int nb0, int nseg,
                                            uint8_t* lds, uint16_t* __restrict__ y, float* __restrict__ yf) {
  DownEpi8<MS, F8WLayout> epi{un, d, nb0, y, yf};
  f8w_stream<MS, LT, false>(rows, I, nseg, lds, epi);
}

// Token-row offsets of the unit's 256 tile rows (source rows in LDS, visible).
__device__ __forceinline__ void f8w_row_offsets(F8WRows& rows, const int* srcrow, int K) {
  rows.kc = K / 128;
#pragma unroll
  for (int q = 0; q < F8W::TL; ++q)
    rows.ot[q] = static_cast<uint32_t>(srcrow[f8w_load_row(q)]) * K + f8w_load_chunk(q) * 16;
}

// The (MS, LT) instance of this wave: LT = 2 token load slots when the block has more than four sub-tiles.
#define F8W_DISPATCH(UNIT, ...)                               \
  do {                                                        \
    const int ms_ = F8WLayout::live(un.nsub);                 \
    if (un.nsub > 4) {                                        \
      if (ms_ == 2) UNIT<2, 2>(__VA_ARGS__);                  \
      else UNIT<1, 2>(__VA_ARGS__);                           \
    } else {                                                  \
      if (ms_ == 1) UNIT<1, 1>(__VA_ARGS__);                  \
      else UNIT<0, 1>(__VA_ARGS__);                           \
    }                                                         \
  } while (0)

__global__ __launch_bounds__(F8W::NT, 1) void ffn_gate_up_fp8w_kernel(
    int d, int I, int E, int n_rows, int a_rows, const int32_t* __restrict__ off, moe_row_mode mode,
    const int32_t* __restrict__ row_src, const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ wgu, const float* __restrict__ wgu_scale, uint8_t* __restrict__ Hq,
    float* __restrict__ Hs, uint8_t* __restrict__ GUq, float* __restrict__ GUs, int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t ldsw[];
  float* swt = reinterpret_cast<float*>(ldsw + F8W::SW_OFF);
  int* srcrow = reinterpret_cast<int*>(ldsw + F8W::SRC_OFF);
  int* cum = reinterpret_cast<int*>(ldsw + F8W::LDS_BYTES);
  __shared__ int wtmp[16];
  const int kc = d / 128, NB = I / 128;
  const int total = build_units_balanced(off, E, n_rows, F8W::MAXSUB, cdiv(NB, kGateUpSegW), cum, wtmp);
  const int tid = threadIdx.x;
  F8WRows rows;
  rows.trs = pipe_rsrc(a, static_cast<uint64_t>(a_rows) * d);
  rows.srs = pipe_rsrc(a_scale, static_cast<uint64_t>(a_rows) * kc * 4);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced<true>(t, off, E, n_rows, F8W::MAXSUB, cum);
    const int nb0 = un.nb * kGateUpSegW, nseg = min(kGateUpSegW, NB - nb0);
    // weight scales of each tile (gate block row nb, up block row I/128 + nb) and the source row of each
    // tile row (rows past the block read any valid row and are never stored)
    const float* sexp = wgu_scale + static_cast<size_t>(un.e) * (2 * I / 128) * kc;
    for (int x = tid; x < nseg * 2 * kc; x += F8W::NT) {
      const int sb = x / kc, c = x - sb * kc, seg = sb >> 1, b = sb & 1;
      swt[(seg * 2 + b) * F8W::MAX_CHUNKS + c] =
          sexp[static_cast<size_t>(b ? I / 128 + nb0 + seg : nb0 + seg) * kc + c];
    }
    if (tid < F8W::BT) {
      int s_first = source_row(mode, row_src, un.m0, un.seg0, a_rows);
      if (s_first < 0) s_first = 0;
      const int sr = tid < un.rows ? source_row(mode, row_src, un.m0 + tid, un.seg0, a_rows) : -1;
      srcrow[tid] = sr < 0 ? s_first : sr;
    }
    __syncthreads();
    f8w_row_offsets(rows, srcrow, d);
    rows.wrs = pipe_rsrc(wgu + (static_cast<size_t>(un.e) * NB + nb0) * F8W::BW * d,
                         static_cast<uint64_t>(nseg) * F8W::BW * d);
    F8W_DISPATCH(gate_up8w_unit, rows, d, I, un, nb0, nseg, ldsw, Hq, Hs, GUq, GUs);
  }
}

__global__ __launch_bounds__(F8W::NT, 1) void ffn_down_fp8w_kernel(int d, int I, int E, int n_rows,
                                                                   const int32_t* __restrict__ off,
                                                                   const uint8_t* __restrict__ Hq,
                                                                   const float* __restrict__ Hs,
                                                                   const uint8_t* __restrict__ wd,
                                                                   const float* __restrict__ wd_scale,
                                                                   uint16_t* __restrict__ y, float* __restrict__ yf,
                                                                   int* __restrict__ q) {
  extern __shared__ __align__(16) uint8_t ldsw[];
  float* swt = reinterpret_cast<float*>(ldsw + F8W::SW_OFF);
  int* srcrow = reinterpret_cast<int*>(ldsw + F8W::SRC_OFF);
  int* cum = reinterpret_cast<int*>(ldsw + F8W::LDS_BYTES);
  __shared__ int wtmp[16];
  const int kc = I / 128, NBF = d / F8W::BW;                 // d % 256 == 0
  const int total = build_units_balanced(off, E, n_rows, F8W::MAXSUB, cdiv(NBF, F8W::MAX_SEG), cum, wtmp);
  const int tid = threadIdx.x;
  F8WRows rows;
  rows.trs = pipe_rsrc(Hq, static_cast<uint64_t>(n_rows) * I);
  rows.srs = pipe_rsrc(Hs, static_cast<uint64_t>(n_rows) * kc * 4);
  __shared__ int tslot;
  int x_off = 0;
  for (int t; (t = unit_queue_next(q, total, x_off, &tslot)) >= 0;) {
    const Unit un = find_unit_balanced<true>(t, off, E, n_rows, F8W::MAXSUB, cum);
    const int nb0 = un.nb * F8W::MAX_SEG, nseg = min(F8W::MAX_SEG, NBF - nb0);
    // weight scales: wave half ww of tile nb covers output columns nb*256 + 128ww .. +127 = block row 2nb + ww
    const float* sexp = wd_scale + static_cast<size_t>(un.e) * (d / 128) * kc;
    for (int x = tid; x < nseg * 2 * kc; x += F8W::NT) {
      const int sb = x / kc, c = x - sb * kc;
      swt[sb * F8W::MAX_CHUNKS + c] = sexp[static_cast<size_t>(2 * nb0 + sb) * kc + c];
    }
    if (tid < F8W::BT) srcrow[tid] = un.m0 + (tid < un.rows ? tid : 0);
    __syncthreads();
    f8w_row_offsets(rows, srcrow, I);
    rows.wrs = pipe_rsrc(wd + (static_cast<size_t>(un.e) * NBF + nb0) * F8W::BW * I,
                         static_cast<uint64_t>(nseg) * F8W::BW * I);
    F8W_DISPATCH(down8w_unit, rows, d, I, un, nb0, nseg, ldsw, y, yf);
  }
}

// The eight-wave kernels take whole token-scale windows (K % 1024), the
// weight-scale table (K / 128 <= MAX_CHUNKS), whole 256-column output tiles
// and the schedule table of up to kMaxExpertsW experts.
static bool f8w_gate_up_fits(const FfnArgs& p) {
  return p.d % 1024 == 0 && p.d / 128 <= F8W::MAX_CHUNKS && p.n_experts <= kMaxExpertsW;
}
static bool f8w_down_fits(const FfnArgs& p) {
  return p.I % 1024 == 0 && p.I / 128 <= F8W::MAX_CHUNKS && p.d % F8W::BW == 0 && p.n_experts <= kMaxExpertsW;
}

static int f8_grid(long long units_upper) {
  long long g = static_cast<long long>(device_cu_count());   // one workgroup per CU
  if (units_upper < g) g = units_upper;
  g = ((g + 7) / 8) * 8;
  return static_cast<int>(g < 8 ? 8 : g);
}

static void f8_set_lds_limits() {
  static std::once_flag once;
  std::call_once(once, [] {
    // ring + weight scales + schedule for up to kMaxExperts8 experts; a refused
    // request must not leave a sticky error
    const int need = P8::LDS_BYTES + 4 * (kMaxExperts8 + 1);
    static_assert(P8::LDS_BYTES + 4 * (kMaxExperts8 + 1) + 64 <= 160 * 1024, "LDS budget");
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_gate_up_fp8_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, need);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_down_fp8_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, need);
    const int need_w = F8W::LDS_BYTES + 4 * (kMaxExpertsW + 1);
    static_assert(F8W::LDS_BYTES + 4 * (kMaxExpertsW + 1) + 128 <= 160 * 1024, "LDS budget");
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_gate_up_fp8w_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, need_w);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_down_fp8w_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, need_w);
    (void)hipGetLastError();
  });
}

hipError_t launch_ffn_fp8_gate_up(const FfnArgs& p, hipStream_t st) {
  if (p.n_experts > kMaxExperts8) return hipErrorInvalidValue;
  f8_set_lds_limits();
  int* q = p.queue;
  if (hipError_t e = launch_queue_reset(q, st); e != hipSuccess) return e;
  if (f8w_gate_up_fits(p)) {
    const size_t lds = F8W::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
    const long long mblocks = p.n_rows / F8W::BT + p.n_experts;
    hipLaunchKernelGGL(ffn_gate_up_fp8w_kernel, dim3(f8_grid(mblocks * cdiv(p.I / 128, kGateUpSegW))),
                       dim3(F8W::NT), lds, st, p.d, p.I, p.n_experts, p.n_rows, p.a_rows, p.offsets, p.mode,
                       p.row_src, static_cast<const uint8_t*>(p.a), p.a_scale, static_cast<const uint8_t*>(p.w_gu),
                       static_cast<const float*>(p.w_gu_scale), static_cast<uint8_t*>(p.h), p.h_scale,
                       static_cast<uint8_t*>(p.gu_cache), p.gu_scale, q);
    return hipGetLastError();
  }
  const size_t lds = P8::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / P8::BT + p.n_experts;
  hipLaunchKernelGGL(ffn_gate_up_fp8_kernel, dim3(f8_grid(mblocks * cdiv(p.I / 128, P8::MAX_SEG))), dim3(P8::NT), lds,
                     st, p.d, p.I,
                     p.n_experts, p.n_rows, p.a_rows, p.offsets, p.mode, p.row_src,
                     static_cast<const uint8_t*>(p.a), p.a_scale, static_cast<const uint8_t*>(p.w_gu), static_cast<const float*>(p.w_gu_scale),
                     static_cast<uint8_t*>(p.h), p.h_scale, static_cast<uint8_t*>(p.gu_cache), p.gu_scale, q);
  return hipGetLastError();
}

hipError_t launch_ffn_fp8_down(const FfnArgs& p, hipStream_t st) {
  if (p.n_experts > kMaxExperts8) return hipErrorInvalidValue;
  f8_set_lds_limits();
  int* q = p.queue;
  if (hipError_t e = launch_queue_reset(q, st); e != hipSuccess) return e;
  if (f8w_down_fits(p)) {
    const size_t lds = F8W::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
    const long long mblocks = p.n_rows / F8W::BT + p.n_experts;
    hipLaunchKernelGGL(ffn_down_fp8w_kernel, dim3(f8_grid(mblocks * cdiv(p.d / F8W::BW, F8W::MAX_SEG))),
                       dim3(F8W::NT), lds, st, p.d, p.I, p.n_experts, p.n_rows, p.offsets,
                       static_cast<const uint8_t*>(p.h), p.h_scale, static_cast<const uint8_t*>(p.w_d),
                       static_cast<const float*>(p.w_d_scale),
                       p.y_dtype == MOE_F32 ? nullptr : static_cast<uint16_t*>(p.y),
                       p.y_dtype == MOE_F32 ? static_cast<float*>(p.y) : nullptr, q);
    return hipGetLastError();
  }
  const size_t lds = P8::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / P8::BT + p.n_experts;
  hipLaunchKernelGGL(ffn_down_fp8_kernel, dim3(f8_grid(mblocks * (cdiv(p.d / P8::BW, P8::MAX_SEG) + 1))), dim3(P8::NT),
                     lds,
                     st, p.d, p.I,
                     p.n_experts, p.n_rows, p.offsets, static_cast<const uint8_t*>(p.h), p.h_scale,
                     static_cast<const uint8_t*>(p.w_d), static_cast<const float*>(p.w_d_scale),
                     p.y_dtype == MOE_F32 ? nullptr : static_cast<uint16_t*>(p.y),
                     p.y_dtype == MOE_F32 ? static_cast<float*>(p.y) : nullptr, q);
  return hipGetLastError();
}

}  // namespace moe
