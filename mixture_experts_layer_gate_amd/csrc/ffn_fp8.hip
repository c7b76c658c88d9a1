// Grouped SwiGLU expert FFN with E4M3 operands ("DeepSeek_V3_Report: Annotation",
// §Fine-Grained Quantization and §Increasing Accumulation Precision; "DeepSeek
// V3 / V4 Infra", V3 FP8 section).
//
// Activations carry one fp32 scale per 1x128 tile (row, K chunk), weights one
// per 128x128 block. The K loop runs one 128-wide chunk at a time: two
// v_mfma_f32_32x32x64_f8f6f4 accumulate the chunk's raw code products into a
// temporary, which is then promoted into the fp32 accumulator with the
// product of the row's activation scale and the block's weight scale -- the
// pages' fp32 promotion every N_C = 128 elements. (gfx950's block-scaled MFMA
// takes power-of-two E8M0 scales per 32 elements, which cannot carry these
// fp32 scales, so the promotion runs on the VALU.)
//
// Tiles: 64 rows x 256 weight rows, four waves of 64 x 64, both operands
// staged through double-buffered LDS. The gate/up tile covers 128 complete H
// columns (each wave 32 gate rows + the matching 32 up rows), so the SwiGLU
// output is re-quantised per 1x128 tile along I in the epilogue.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "sched.h"

namespace moe {

struct F8Tile {
  static constexpr int BM = 64, BN = 256, NT = 256, TM = 2, TN = 2;
  static constexpr int CK = 128;            // K chunk = scale group
  static constexpr int LDB = CK + 16;       // padded LDS row in bytes
  static constexpr int AC = BM * (CK / 16) / NT;   // 16-byte A chunks per thread (2)
  static constexpr int BC = BN * (CK / 16) / NT;   // 16-byte B chunks per thread (8)
  static constexpr int STAGE = (BM + BN) * LDB;    // bytes per LDS stage
  static constexpr int LDS_BYTES = 2 * STAGE + 2 * BM * 4;  // + activation scales
};

__device__ __forceinline__ int f8_row(int tid, int j) { return (tid + F8Tile::NT * j) >> 3; }
__device__ __forceinline__ int f8_col(int tid, int j) { return ((tid + F8Tile::NT * j) & 7) * 16; }

// acc[i][j] (+)= sum over K chunks c of sa[row, c] * sw[j, c] * (A_c . B_c^T)
//  pa[q]      : this thread's A chunk byte pointers (row start + column), or null
//  pb[q]      : this thread's B chunk byte pointers
//  sa_ptr     : for threads tid < BM, the row's scale pointer (stride 1 per chunk), or null
//  sw_ptr[j]  : this wave's weight-scale pointers for sub-tile column j (stride 1 per chunk)
__device__ __forceinline__ void f8_mainloop(const uint8_t* const (&pa)[F8Tile::AC], const uint8_t* const (&pb)[F8Tile::BC],
                                            const float* sa_ptr, const float* const (&sw_ptr)[F8Tile::TN], int K,
                                            uint8_t* lds, f32x16 (&acc)[F8Tile::TM][F8Tile::TN]) {
  using G = F8Tile;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  float* sas = reinterpret_cast<float*>(lds + 2 * G::STAGE);   // [2][BM]
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 ra[G::AC], rb[G::BC];
  float rs = 0.0f;
  const int nk = K / G::CK;

  auto stage_of = [&](int buf) { return lds + buf * G::STAGE; };
#pragma unroll
  for (int q = 0; q < G::AC; ++q) ra[q] = pa[q] ? *reinterpret_cast<const u32x4*>(pa[q]) : z;
#pragma unroll
  for (int q = 0; q < G::BC; ++q) rb[q] = *reinterpret_cast<const u32x4*>(pb[q]);
  if (tid < G::BM) rs = sa_ptr ? sa_ptr[0] : 0.0f;
  {
    uint8_t* st = stage_of(0);
#pragma unroll
    for (int q = 0; q < G::AC; ++q) *reinterpret_cast<u32x4*>(st + f8_row(tid, q) * G::LDB + f8_col(tid, q)) = ra[q];
#pragma unroll
    for (int q = 0; q < G::BC; ++q)
      *reinterpret_cast<u32x4*>(st + (G::BM + f8_row(tid, q)) * G::LDB + f8_col(tid, q)) = rb[q];
    if (tid < G::BM) sas[tid] = rs;
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = (kt + 1) * G::CK;
#pragma unroll
      for (int q = 0; q < G::AC; ++q) ra[q] = pa[q] ? *reinterpret_cast<const u32x4*>(pa[q] + k0) : z;
#pragma unroll
      for (int q = 0; q < G::BC; ++q) rb[q] = *reinterpret_cast<const u32x4*>(pb[q] + k0);
      if (tid < G::BM) rs = sa_ptr ? sa_ptr[kt + 1] : 0.0f;
    }
    const uint8_t* st = stage_of(buf);
    float swj[G::TN];
#pragma unroll
    for (int j = 0; j < G::TN; ++j) swj[j] = sw_ptr[j][kt];
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      // A fragments of M sub-tile i for the two 64-wide halves of the chunk
      i32x8 af[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* p = st + (i * 32 + (lane & 31)) * G::LDB + 64 * s + 32 * h;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
        af[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // row scales of this lane's 16 accumulator rows
      float sr[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(&sas[buf * G::BM + i * 32 + 8 * q + 4 * h]);
        sr[4 * q + 0] = v4.x; sr[4 * q + 1] = v4.y; sr[4 * q + 2] = v4.z; sr[4 * q + 3] = v4.w;
      }
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        f32x16 t;
#pragma unroll
        for (int v = 0; v < 16; ++v) t[v] = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint8_t* p = st + (G::BM + 64 * w + 32 * j + (lane & 31)) * G::LDB + 64 * s + 32 * h;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
          const i32x8 bf = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s], bf, t, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(t[v], sr[v] * swj[j], acc[i][j][v]);
      }
    }
    if (more) {
      uint8_t* sn = stage_of(buf ^ 1);
#pragma unroll
      for (int q = 0; q < G::AC; ++q) *reinterpret_cast<u32x4*>(sn + f8_row(tid, q) * G::LDB + f8_col(tid, q)) = ra[q];
#pragma unroll
      for (int q = 0; q < G::BC; ++q)
        *reinterpret_cast<u32x4*>(sn + (G::BM + f8_row(tid, q)) * G::LDB + f8_col(tid, q)) = rb[q];
      if (tid < G::BM) sas[(buf ^ 1) * G::BM + tid] = rs;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ int f8_acc_row(int i, int v) {
  const int lane = threadIdx.x & 63;
  return i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__global__ __launch_bounds__(F8Tile::NT) void ffn_gate_up_fp8_kernel(
    int d, int I, int E, int n_rows, int a_rows, const int32_t* __restrict__ off, moe_row_mode mode,
    const int32_t* __restrict__ row_src, const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ wgu, const float* __restrict__ wgu_scale, uint8_t* __restrict__ Hq,
    float* __restrict__ Hs) {
  using G = F8Tile;
  extern __shared__ __align__(16) uint8_t lds_f8[];
  int* cum = reinterpret_cast<int*>(lds_f8 + G::LDS_BYTES);
  __shared__ int wtmp[16];
  __shared__ float row_amax[4][G::BM];
  const int NB = I / 128;
  const int total = build_units(off, E, n_rows, G::BM, NB, cum, wtmp);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kc = d / 128;
  for (int t = xcd_virtual_block(); t < total; t += gridDim.x) {
    const Unit un = find_unit(t, off, E, n_rows, G::BM, cum);
    const uint8_t* pa[G::AC];
#pragma unroll
    for (int q = 0; q < G::AC; ++q) {
      const int r = f8_row(tid, q);
      const int sr = r < un.rows ? source_row(mode, row_src, un.m0 + r, un.seg0, a_rows) : -1;
      pa[q] = sr >= 0 ? a + static_cast<size_t>(sr) * d + f8_col(tid, q) : nullptr;
    }
    const float* sa_ptr = nullptr;
    if (tid < G::BM && tid < un.rows) {
      const int sr = source_row(mode, row_src, un.m0 + tid, un.seg0, a_rows);
      if (sr >= 0) sa_ptr = a_scale + static_cast<size_t>(sr) * kc;
    }
    const uint8_t* wexp = wgu + static_cast<size_t>(un.e) * 2 * I * d;
    const uint8_t* pb[G::BC];
#pragma unroll
    for (int q = 0; q < G::BC; ++q) {
      const int rb = f8_row(tid, q);
      const int hcol = un.nb * 128 + (rb >> 6) * 32 + (rb & 31);
      const int wrow = ((rb >> 5) & 1) ? I + hcol : hcol;
      pb[q] = wexp + static_cast<size_t>(wrow) * d + f8_col(tid, q);
    }
    const float* sexp = wgu_scale + static_cast<size_t>(un.e) * (2 * I / 128) * kc;
    const float* sw_ptr[G::TN] = {sexp + static_cast<size_t>(un.nb) * kc,
                                  sexp + static_cast<size_t>(I / 128 + un.nb) * kc};
    f32x16 acc[G::TM][G::TN];
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    f8_mainloop(pa, pb, sa_ptr, sw_ptr, d, lds_f8, acc);

    // SwiGLU, then 1x128 quantisation of H along I (this tile owns 128 columns)
    float hv[G::TM][16];
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) hv[i][v] = silu(acc[i][0][v]) * acc[i][1][v];
    // per-row max over this wave's 32 columns: rows (i, v) live in lanes with equal lane/32
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = __builtin_fabsf(hv[i][v]);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
        if ((lane & 31) == 0) row_amax[w][f8_acc_row(i, v)] = x;
      }
    __syncthreads();
    const int col = un.nb * 128 + 32 * w + (lane & 31);
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = f8_acc_row(i, v);
        const float amax = fmaxf(fmaxf(row_amax[0][r], row_amax[1][r]), fmaxf(row_amax[2][r], row_amax[3][r]));
        if (r < un.rows) {
          const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
          Hq[static_cast<size_t>(un.m0 + r) * I + col] = static_cast<uint8_t>(f32_to_e4m3(hv[i][v] * inv));
          if (w == 0 && (lane & 31) == 0) Hs[static_cast<size_t>(un.m0 + r) * NB + un.nb] = amax > 0.0f ? amax / kE4M3Max : 1.0f;
        }
      }
    __syncthreads();
  }
}

__global__ __launch_bounds__(F8Tile::NT) void ffn_down_fp8_kernel(int d, int I, int E, int n_rows,
                                                                  const int32_t* __restrict__ off,
                                                                  const uint8_t* __restrict__ Hq,
                                                                  const float* __restrict__ Hs,
                                                                  const uint8_t* __restrict__ wd,
                                                                  const float* __restrict__ wd_scale,
                                                                  uint16_t* __restrict__ y) {
  using G = F8Tile;
  extern __shared__ __align__(16) uint8_t lds_f8[];
  int* cum = reinterpret_cast<int*>(lds_f8 + G::LDS_BYTES);
  __shared__ int wtmp[16];
  const int NB = d / G::BN;
  const int total = build_units(off, E, n_rows, G::BM, NB, cum, wtmp);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kc = I / 128;
  for (int t = xcd_virtual_block(); t < total; t += gridDim.x) {
    const Unit un = find_unit(t, off, E, n_rows, G::BM, cum);
    const uint8_t* pa[G::AC];
#pragma unroll
    for (int q = 0; q < G::AC; ++q) {
      const int r = f8_row(tid, q);
      pa[q] = r < un.rows ? Hq + static_cast<size_t>(un.m0 + r) * I + f8_col(tid, q) : nullptr;
    }
    const float* sa_ptr = (tid < G::BM && tid < un.rows) ? Hs + static_cast<size_t>(un.m0 + tid) * kc : nullptr;
    const uint8_t* wexp = wd + static_cast<size_t>(un.e) * d * I;
    const uint8_t* pb[G::BC];
#pragma unroll
    for (int q = 0; q < G::BC; ++q) {
      const int n = un.nb * G::BN + f8_row(tid, q);
      pb[q] = wexp + static_cast<size_t>(n) * I + f8_col(tid, q);
    }
    // wave w covers output columns nb*256 + 64w .. +63: one 128-row weight block row
    const float* sexp = wd_scale + static_cast<size_t>(un.e) * (d / 128) * kc;
    const int brow = (un.nb * G::BN + 64 * w) / 128;
    const float* sw_ptr[G::TN] = {sexp + static_cast<size_t>(brow) * kc, sexp + static_cast<size_t>(brow) * kc};
    f32x16 acc[G::TM][G::TN];
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    f8_mainloop(pa, pb, sa_ptr, sw_ptr, I, lds_f8, acc);
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int n = un.nb * G::BN + 64 * w + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = f8_acc_row(i, v);
          if (r < un.rows) y[static_cast<size_t>(un.m0 + r) * d + n] = f32_to_bf16(acc[i][j][v]);
        }
      }
  }
}

static int f8_grid(long long units_upper) {
  long long g = static_cast<long long>(device_cu_count());   // one 90 KB-LDS workgroup per CU
  if (units_upper < g) g = units_upper;
  g = ((g + 7) / 8) * 8;
  return static_cast<int>(g < 8 ? 8 : g);
}

static void f8_set_lds_limits() {
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_gate_up_fp8_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 120 * 1024);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ffn_down_fp8_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 120 * 1024);
    (void)hipGetLastError();
  });
}

hipError_t launch_ffn_fp8_gate_up(const FfnArgs& p, hipStream_t st) {
  using G = F8Tile;
  f8_set_lds_limits();
  const size_t lds = G::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / G::BM + p.n_experts;
  hipLaunchKernelGGL(ffn_gate_up_fp8_kernel, dim3(f8_grid(mblocks * (p.I / 128))), dim3(G::NT), lds, st, p.d, p.I,
                     p.n_experts, p.n_rows, p.a_rows, p.offsets, p.mode, p.row_src,
                     static_cast<const uint8_t*>(p.a), p.a_scale, static_cast<const uint8_t*>(p.w_gu), p.w_gu_scale,
                     static_cast<uint8_t*>(p.h), p.h_scale);
  return hipGetLastError();
}

hipError_t launch_ffn_fp8_down(const FfnArgs& p, hipStream_t st) {
  using G = F8Tile;
  f8_set_lds_limits();
  const size_t lds = G::LDS_BYTES + sizeof(int) * (p.n_experts + 1);
  const long long mblocks = p.n_rows / G::BM + p.n_experts;
  hipLaunchKernelGGL(ffn_down_fp8_kernel, dim3(f8_grid(mblocks * (p.d / G::BN))), dim3(G::NT), lds, st, p.d, p.I,
                     p.n_experts, p.n_rows, p.offsets, static_cast<const uint8_t*>(p.h), p.h_scale,
                     static_cast<const uint8_t*>(p.w_d), p.w_d_scale, static_cast<uint16_t*>(p.y));
  return hipGetLastError();
}

}  // namespace moe
