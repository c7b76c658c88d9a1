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

template <class X>
__global__ __launch_bounds__(256) void quantize_rows_kernel(long long n_tiles, const X* __restrict__ x,
                                                            uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int l = threadIdx.x & 63;
  for (long long t = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) >> 6; t < n_tiles;
       t += static_cast<long long>(gridDim.x) * 4) {
    const size_t o = static_cast<size_t>(t) * 128 + 2 * l;             // row-major: tile t = row t / (C/128)
    const float2 v = load_pair(x + o);
    const float a = v.x, b = v.y;
    float m = fmaxf(__builtin_fabsf(a), __builtin_fabsf(b));
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    const float inv = m > 0.0f ? kE4M3Max / m : 0.0f;
    *reinterpret_cast<uint16_t*>(codes + o) =
        static_cast<uint16_t>(f32_to_e4m3(a * inv) | (f32_to_e4m3(b * inv) << 8));
    if (l == 0) scales[t] = m > 0.0f ? m / kE4M3Max : 1.0f;
  }
}

// Elementwise over [n_rows, I]: G, U dequantised from the cache; dG = dh U SiLU'(G), dU = dh SiLU(G), h = SiLU(G) U.
__global__ __launch_bounds__(256) void swiglu_backward8_kernel(long long n, int I, const float* __restrict__ dh,
                                                               const uint8_t* __restrict__ guq,
                                                               const float* __restrict__ gus,
                                                               float* __restrict__ dgu, float* __restrict__ h) {
  const int kc = 2 * I / 128;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long r = i / I;
    const int c = static_cast<int>(i - r * I);
    const float g = e4m3_value(guq[r * 2 * I + c]) * gus[r * kc + c / 128];
    const float up = e4m3_value(guq[r * 2 * I + I + c]) * gus[r * kc + (I + c) / 128];
    const float dv = dh[i];
    const float sg = 1.0f / (1.0f + expf(-g));
    const float si = g * sg;
    dgu[r * 2 * I + c] = dv * up * sg * (1.0f + g * (1.0f - sg));
    dgu[r * 2 * I + I + c] = dv * si;
    h[i] = si * up;
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

// A block per (128-row block, 256 columns): thread = column. The source is bf16 rows of x (row r, DIRECT) or,
// with GATHERED, E4M3 codes with their 1x128 fp32 scales at the row's source row (row_src / segment / direct).
template <bool GATHERED, class X>
__global__ __launch_bounds__(256) void requant_cols_kernel(int C, int E, int n_rows, const int32_t* __restrict__ off,
                                                           const int* __restrict__ pre, moe_row_mode mode,
                                                           const int32_t* __restrict__ row_src, int a_rows,
                                                           const X* __restrict__ x,
                                                           const uint8_t* __restrict__ xq,
                                                           const float* __restrict__ xs, uint16_t* __restrict__ out) {
  const int ncc = cdiv(C, 256);
  const int j = blockIdx.x / ncc, c = (blockIdx.x % ncc) * 256 + threadIdx.x;
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
  auto value = [&](int r) -> float {
    if (!GATHERED) return load_one(x + static_cast<size_t>(r) * C + c);
    const int sr = source_row(mode, row_src, r, lo, a_rows);
    if (sr < 0) return 0.0f;
    return e4m3_value(xq[static_cast<size_t>(sr) * C + c]) * xs[static_cast<size_t>(sr) * (C / 128) + c / 128];
  };
  float amax = 0.0f;
  for (int r = b0; r < b1; ++r) amax = fmaxf(amax, __builtin_fabsf(value(r)));
  const int n = amax > 0.0f ? pow2_scale_exp(amax) : 0;
  for (int r = b0; r < b1; ++r) {
    const float q = amax > 0.0f ? e4m3_value(f32_to_e4m3(__builtin_ldexpf(value(r), -n))) : 0.0f;
    out[static_cast<size_t>(r) * C + c] = f32_to_bf16(__builtin_ldexpf(q, n));
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
  const dim3 g(static_cast<unsigned>(grid_cap8(cdiv(tiles, 4))));
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
  const long long n = n_rows * I;
  hipLaunchKernelGGL(swiglu_backward8_kernel, dim3(static_cast<unsigned>(grid_cap8((n + 255) / 256))), dim3(256), 0,
                     st, n, I, static_cast<const float*>(dh), static_cast<const uint8_t*>(guq), gus,
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
  const long long blocks = (static_cast<long long>(n_rows) / 128 + E) * cdiv(C, 256);   // covers every 128-row block
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
