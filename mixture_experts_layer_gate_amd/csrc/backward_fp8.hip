// The FP8 recipe of the layer backward ("DeepSeek_V3_Report: Annotation", FP8
// framework: all three GEMMs of a linear layer in FP8; the SwiGLU inputs cached
// as fine-grained FP8 tiles and the SwiGLU output recomputed in the backward;
// the activations re-tiled from 1x128 to 128x1 for the weight-gradient GEMM).
// dy comes from the combine backward in bf16 (the combine stays in BF16 in
// both passes); the GEMM output dh and the SwiGLU backward's dG, dU, h are
// fp32 (the pages' GEMMs output BF16 or FP32):
//
//  transpose_rows:    W [R, C] -> W^T [C, R] bf16 (row-major), so the transposed
//                     weights of the input-gradient GEMMs quantise into the
//                     same 128x128 blocks (one scale per block either way)
//  quantize_rows:     x [n, C] bf16 / fp32 -> E4M3 codes + one fp32 scale per 1x128
//                     tile (the forward's activation rule): the input of an
//                     FP8 input-gradient GEMM
//  swiglu_backward8:  dh and the cached E4M3 [G, U] tiles -> dG, dU, and the
//                     recomputed h = SiLU(G) U, fp32
//  requant_cols:      the 128x1 re-tiling of a weight-gradient operand: per
//                     column and block of 128 consecutive rows of an expert
//                     (from its first row) one power-of-two scale; the E4M3
//                     values times that scale are written back as bf16, which
//                     holds them exactly, so the weight-gradient GEMM consumes
//                     exactly the re-tiled FP8 operand
#include "common.h"
#include "launch.h"
#include "sched.h"

namespace moe {

namespace {

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code), 0);
}

// The smallest power of two >= fl32(amax / 448) as 2^n (amax > 0).
__device__ __forceinline__ int pow2_scale_exp(float amax) {
  int e;
  const float m = __builtin_frexpf(amax / kE4M3Max, &e);   // v = m 2^e, 0.5 <= m < 1
  return m == 0.5f ? e - 1 : e;
}

}  // namespace

// 64 x 64 tiles through LDS; a block per (tile, matrix).
__global__ __launch_bounds__(256) void transpose_rows_kernel(int R, int C, const uint16_t* __restrict__ w,
                                                             uint16_t* __restrict__ out) {
  __shared__ uint16_t t[64][66];
  const int tc = blockIdx.x, tr = blockIdx.y;
  const size_t mat = blockIdx.z;
  const uint16_t* src = w + mat * R * C;
  uint16_t* dst = out + mat * R * C;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    t[r][c] = src[static_cast<size_t>(tr * 64 + r) * C + tc * 64 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i >> 6, r = i & 63;
    dst[static_cast<size_t>(tc * 64 + c) * R + tr * 64 + r] = t[r][c];
  }
}

// One wavefront per (row, 128-column tile), two values per lane (X: bf16 as uint16_t, or float).
__device__ __forceinline__ float2 load_pair(const uint16_t* p) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u));
}
__device__ __forceinline__ float2 load_pair(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ float load_one(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_one(const float* p) { return *p; }

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// 16 lanes per (row, 128-column tile), 8 consecutive values per lane.
template <class X>
__global__ __launch_bounds__(256) void quantize_rows_kernel(long long n_tiles, const X* __restrict__ x,
                                                            uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int l = threadIdx.x & 15;
  for (long long t = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) >> 4; t < n_tiles;
       t += static_cast<long long>(gridDim.x) * 16) {
    const size_t o = static_cast<size_t>(t) * 128 + 8 * l;             // row-major: tile t = row t / (C/128)
    float v[8];
    load8(x + o, v);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[i]));
#pragma unroll
    for (int s = 8; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 16));
    const float inv = m > 0.0f ? kE4M3Max / m : 0.0f;
    uint32_t c[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i >> 2] |= f32_to_e4m3(v[i] * inv) << (8 * (i & 3));
    *reinterpret_cast<uint2*>(codes + o) = make_uint2(c[0], c[1]);
    if (l == 0) scales[t] = m > 0.0f ? m / kE4M3Max : 1.0f;
  }
}

// Elementwise over [n_rows, I], 4 consecutive columns per thread: G, U dequantised from the cache;
// dG = dh U SiLU'(G), dU = dh SiLU(G), h = SiLU(G) U.
__global__ __launch_bounds__(256) void swiglu_backward8_kernel(long long n4, int I, const float* __restrict__ dh,
                                                               const uint8_t* __restrict__ guq,
                                                               const float* __restrict__ gus,
                                                               float* __restrict__ dgu, float* __restrict__ h) {
  const int kc = 2 * I / 128, I4 = I / 4;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long r = i / I4;
    const int c = static_cast<int>(i - r * I4) * 4;
    const uint32_t qg = *reinterpret_cast<const uint32_t*>(guq + r * 2 * I + c);
    const uint32_t qu = *reinterpret_cast<const uint32_t*>(guq + r * 2 * I + I + c);
    const float sgs = gus[r * kc + c / 128], sus = gus[r * kc + (I + c) / 128];
    const float4 dv4 = *reinterpret_cast<const float4*>(dh + r * I + c);
    const float dv[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
    float dg[4], du[4], hv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float g = e4m3_value((qg >> (8 * k)) & 0xFFu) * sgs;
      const float up = e4m3_value((qu >> (8 * k)) & 0xFFu) * sus;
      const float sg = 1.0f / (1.0f + expf(-g));
      const float si = g * sg;
      dg[k] = dv[k] * up * sg * (1.0f + g * (1.0f - sg));
      du[k] = dv[k] * si;
      hv[k] = si * up;
    }
    *reinterpret_cast<float4*>(dgu + r * 2 * I + c) = make_float4(dg[0], dg[1], dg[2], dg[3]);
    *reinterpret_cast<float4*>(dgu + r * 2 * I + I + c) = make_float4(du[0], du[1], du[2], du[3]);
    *reinterpret_cast<float4*>(h + r * I + c) = make_float4(hv[0], hv[1], hv[2], hv[3]);
  }
}

// pre[e] = number of 128-row blocks of experts 0 .. e-1 (one thread; E + 1 entries).
__global__ void row_block_prefix_kernel(int E, int n_rows, const int32_t* __restrict__ off, int* __restrict__ pre) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int acc = 0;
  for (int e = 0; e < E; ++e) {
    pre[e] = acc;
    const int lo = clampi(off[e], 0, n_rows), hi = clampi(off[e + 1], lo, n_rows);
    acc += cdiv(hi - lo, 128);
  }
  pre[E] = acc;
}

// A block per (128-row block, 1024 columns): each thread 4 adjacent columns. The source is bf16 / fp32 rows of x
// (row r, DIRECT) or, with GATHERED, E4M3 codes with their 1x128 fp32 scales at the row's source row.
__device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

template <bool GATHERED, class X>
__global__ __launch_bounds__(256) void requant_cols_kernel(int C, int E, int n_rows, const int32_t* __restrict__ off,
                                                           const int* __restrict__ pre, moe_row_mode mode,
                                                           const int32_t* __restrict__ row_src, int a_rows,
                                                           const X* __restrict__ x,
                                                           const uint8_t* __restrict__ xq,
                                                           const float* __restrict__ xs, uint16_t* __restrict__ out) {
  const int ncc = cdiv(C, 1024);
  const int j = blockIdx.x / ncc, c = (blockIdx.x % ncc) * 1024 + 4 * threadIdx.x;
  if (j >= pre[E]) return;
  int lo_e = 0, hi_e = E;                               // the expert e with pre[e] <= j < pre[e + 1]
  while (hi_e - lo_e > 1) {
    const int mid = (lo_e + hi_e) >> 1;
    if (pre[mid] <= j) lo_e = mid;
    else hi_e = mid;
  }
  const int e = lo_e;
  const int lo = clampi(off[e], 0, n_rows), hi = clampi(off[e + 1], lo, n_rows);
  const int b0 = lo + 128 * (j - pre[e]), b1 = min(b0 + 128, hi);
  if (c >= C) return;
  auto values = [&](int r, float (&v)[4]) {
    if (!GATHERED) {
      load4(x + static_cast<size_t>(r) * C + c, v);
      return;
    }
    const int sr = source_row(mode, row_src, r, lo, a_rows);
    if (sr < 0) {
      v[0] = v[1] = v[2] = v[3] = 0.0f;
      return;
    }
    const uint32_t q = *reinterpret_cast<const uint32_t*>(xq + static_cast<size_t>(sr) * C + c);
    const float sc = xs[static_cast<size_t>(sr) * (C / 128) + c / 128];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = e4m3_value((q >> (8 * i)) & 0xFFu) * sc;
  };
  float amax[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r = b0; r < b1; ++r) {
    float v[4];
    values(r, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) amax[i] = fmaxf(amax[i], __builtin_fabsf(v[i]));
  }
  int n[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) n[i] = amax[i] > 0.0f ? pow2_scale_exp(amax[i]) : 0;
  for (int r = b0; r < b1; ++r) {
    float v[4];
    values(r, v);
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = amax[i] > 0.0f ? __builtin_ldexpf(e4m3_value(f32_to_e4m3(__builtin_ldexpf(v[i], -n[i]))), n[i]) : 0.0f;
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(r) * C + c) = make_uint2(pack_bf16x2(o[0], o[1]),
                                                                                 pack_bf16x2(o[2], o[3]));
  }
}

static long long grid_cap8(long long blocks) {
  const long long cap = static_cast<long long>(device_cu_count()) * 16;
  return blocks > cap ? cap : (blocks < 1 ? 1 : blocks);
}

hipError_t launch_transpose_rows_bf16(int n_mats, int rows, int cols, const void* w, void* out, hipStream_t st) {
  hipLaunchKernelGGL(transpose_rows_kernel, dim3(cols / 64, rows / 64, n_mats), dim3(256), 0, st, rows, cols,
                     static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_quantize_rows(long long n_rows, int cols, const void* x, bool f32_in, void* codes, float* scales,
                                hipStream_t st) {
  const long long tiles = n_rows * (cols / 128);
  const dim3 g(static_cast<unsigned>(grid_cap8(cdiv(tiles, 16))));
  if (f32_in)
    hipLaunchKernelGGL(quantize_rows_kernel<float>, g, dim3(256), 0, st, tiles, static_cast<const float*>(x),
                       static_cast<uint8_t*>(codes), scales);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, g, dim3(256), 0, st, tiles, static_cast<const uint16_t*>(x),
                       static_cast<uint8_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward8(long long n_rows, int I, const void* dh, const void* guq, const float* gus,
                                   void* dgu, void* h, hipStream_t st) {
  const long long n4 = n_rows * I / 4;
  hipLaunchKernelGGL(swiglu_backward8_kernel, dim3(static_cast<unsigned>(grid_cap8((n4 + 255) / 256))), dim3(256), 0,
                     st, n4, I, static_cast<const float*>(dh), static_cast<const uint8_t*>(guq), gus,
                     static_cast<float*>(dgu), static_cast<float*>(h));
  return hipGetLastError();
}

hipError_t launch_row_block_prefix(int E, int n_rows, const int32_t* off, int* pre, hipStream_t st) {
  hipLaunchKernelGGL(row_block_prefix_kernel, dim3(1), dim3(64), 0, st, E, n_rows, off, pre);
  return hipGetLastError();
}

hipError_t launch_requant_cols(int C, int E, int n_rows, const int32_t* off, const int* pre, moe_row_mode mode,
                               const int32_t* row_src, int a_rows, const void* x, bool f32_in, const void* xq,
                               const float* xs, void* out, hipStream_t st) {
  const long long blocks = (static_cast<long long>(n_rows) / 128 + E) * cdiv(C, 1024);  // covers every 128-row block
  const dim3 g(static_cast<unsigned>(blocks));
  uint16_t* o = static_cast<uint16_t*>(out);
  if (xq != nullptr)
    hipLaunchKernelGGL((requant_cols_kernel<true, float>), g, dim3(256), 0, st, C, E, n_rows, off, pre, mode, row_src,
                       a_rows, nullptr, static_cast<const uint8_t*>(xq), xs, o);
  else if (f32_in)
    hipLaunchKernelGGL((requant_cols_kernel<false, float>), g, dim3(256), 0, st, C, E, n_rows, off, pre,
                       MOE_ROWS_DIRECT, nullptr, n_rows, static_cast<const float*>(x), nullptr, nullptr, o);
  else
    hipLaunchKernelGGL((requant_cols_kernel<false, uint16_t>), g, dim3(256), 0, st, C, E, n_rows, off, pre,
                       MOE_ROWS_DIRECT, nullptr, n_rows, static_cast<const uint16_t*>(x), nullptr, nullptr, o);
  return hipGetLastError();
}

}  // namespace moe
