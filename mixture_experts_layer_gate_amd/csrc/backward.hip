// Backward of the MoE layer: the small kernels around the expert GEMMs
// ("DeepSeek_V3_Report: Annotation", eq. (12)-(15); the FP8 framework's
// mixed-precision and low-precision-activation sections: the gating module
// and the combine stay in high precision, weight gradients in fp32, and the
// SwiGLU output is recomputed in the backward from its cached inputs).
//
//  combine_backward:  dy rows = g_tk * d_out[t] (routed), d_out[t] (shared);
//                     d_gate[t, k] = d_out[t] . y[row_of(t, k)]
//  route_backward:    ds_k = (dg_k - sum_j g_j dg_j) / S over the selected
//                     experts (S = sum of their s), dz = ds s (1 - s);
//                     du_router[t] = sum_k dz_tk e_{idx_tk};
//                     d_centroids[e] = sum over e's rows of dz * u[token]
//  swiglu_backward:   from dh and the cached G, U: dG = dh U SiLU'(G),
//                     dU = dh SiLU(G), and h = SiLU(G) U for the weight gradient
//  input_grad:        du[t] = d_out[t] + du_router[t] + sum_k da[row_of(t, k)]
//                     + sum_s da[T K + s T + t]
//  transpose_tile:    W [R, C] -> W^T [C, R] in the tiled bf16 layout (the input
//                     gradient GEMMs contract over W's rows)
// Every sum runs in a fixed order in fp32: the results are deterministic.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// DY: uint16_t (bf16 rows) or float (fp32 rows).
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&f)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                                            pack_bf16x2(f[6], f[7]));
}
__device__ __forceinline__ void store8(float* p, const float (&f)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// One wavefront per token, 8 consecutive columns per lane and step (16-byte loads).
template <class DY>
__global__ __launch_bounds__(256) void combine_backward_kernel(int T, int d, int K, int Ns, const uint16_t* __restrict__ dout,
                                                               const uint16_t* __restrict__ y,
                                                               const int32_t* __restrict__ row_of,
                                                               const float* __restrict__ gate, DY* __restrict__ dy,
                                                               float* __restrict__ dgate, int n_rows) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + w; t < T; t += gridDim.x * 4) {
    const uint16_t* o = dout + static_cast<size_t>(t) * d;
    for (int k = 0; k < K; ++k) {
      const int r = row_of[static_cast<size_t>(t) * K + k];
      const bool ok = r >= 0 && r < n_rows;
      const float g = gate[static_cast<size_t>(t) * K + k];
      float dot = 0.0f;
      if (ok) {
        const uint16_t* yr = y + static_cast<size_t>(r) * d;
        DY* dr = dy + static_cast<size_t>(r) * d;
        for (int c = 8 * l; c < d; c += 512) {
          float of[8], yf[8], df[8];
          unpack8(*reinterpret_cast<const uint4*>(o + c), of);
          unpack8(*reinterpret_cast<const uint4*>(yr + c), yf);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            dot = fmaf(of[i], yf[i], dot);
            df[i] = g * of[i];
          }
          store8(dr + c, df);
        }
      }
#pragma unroll
      for (int s = 32; s > 0; s >>= 1) dot += __shfl_xor(dot, s, 64);
      if (l == 0) dgate[static_cast<size_t>(t) * K + k] = ok ? dot : 0.0f;
    }
    for (int s = 0; s < Ns; ++s) {
      DY* dr = dy + (static_cast<size_t>(T) * K + static_cast<size_t>(s) * T + t) * d;
      for (int c = 8 * l; c < d; c += 512) {
        float of[8];
        unpack8(*reinterpret_cast<const uint4*>(o + c), of);
        store8(dr + c, of);
      }
    }
  }
}

// One wavefront per token: dz over the token's K picks (lanes 0..K-1), then
// du_router[t] = sum_k dz_k e_{idx_k} (lanes over d, picks in slot order), and
// dz per permuted row for the centroid gradient.
__global__ __launch_bounds__(256) void route_backward_token_kernel(int T, int d, int N, int K, int act_bf16,
                                                                   const void* __restrict__ cent,
                                                                   const float* __restrict__ scores,
                                                                   const int32_t* __restrict__ idx,
                                                                   const float* __restrict__ dgate,
                                                                   const int32_t* __restrict__ row_of,
                                                                   float* __restrict__ du_router,
                                                                   float* __restrict__ dz_row) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + w; t < T; t += gridDim.x * 4) {
    const int e = l < K ? idx[static_cast<size_t>(t) * K + l] : -1;
    const bool ok = e >= 0 && e < N;
    const float s = ok ? scores[static_cast<size_t>(t) * N + e] : 0.0f;
    const float dg = ok ? dgate[static_cast<size_t>(t) * K + l] : 0.0f;
    float S = 0.0f, gdg = 0.0f;                       // slot order, the same sums on every lane
    for (int j = 0; j < K; ++j) S += __shfl(s, j, 64);
    for (int j = 0; j < K; ++j) gdg += (__shfl(s, j, 64) / S) * __shfl(dg, j, 64);
    const float dz = ok ? (dg - gdg) / S * s * (1.0f - s) : 0.0f;
    if (l < K) {
      const int r = row_of[static_cast<size_t>(t) * K + l];
      if (r >= 0 && r < T * K) dz_row[r] = dz;
    }
    float* du = du_router + static_cast<size_t>(t) * d;
    int es[16];                                              // the picks, read by every lane before the column loop
    float dzs[16];                                           // (K <= 16), so no shuffle runs under a partial mask
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      es[j] = __shfl(e, j < K ? j : 0, 64);
      dzs[j] = __shfl(dz, j < K ? j : 0, 64);
    }
    for (int c = 8 * l; c < d; c += 512) {                   // 8 consecutive columns per lane
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j >= K) break;
        const int ej = es[j];
        const float dzj = dzs[j];
        if (ej >= 0 && ej < N) {
          const size_t off = static_cast<size_t>(ej) * d + c;
          float ev[8];
          if (act_bf16) {
            unpack8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(cent) + off), ev);
          } else {
            const float4 a = reinterpret_cast<const float4*>(static_cast<const float*>(cent) + off)[0];
            const float4 b = reinterpret_cast<const float4*>(static_cast<const float*>(cent) + off)[1];
            ev[0] = a.x; ev[1] = a.y; ev[2] = a.z; ev[3] = a.w; ev[4] = b.x; ev[5] = b.y; ev[6] = b.z; ev[7] = b.w;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(dzj, ev[i], acc[i]);
        }
      }
      store8(du + c, acc);
    }
  }
}

// d_centroids[e][c] = sum over the rows r of expert e of dz_row[r] * u[perm_token[r]][c]; a block per (expert,
// 256 columns). Four rows are loaded at a time into four partial sums (rows r = 4i + j go to sum j), added in the
// order 0..3 at the end: a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void centroid_grad_kernel(int T, int d, int N, int n_rows, int act_bf16,
                                                            const void* __restrict__ u,
                                                            const int32_t* __restrict__ off,
                                                            const int32_t* __restrict__ perm_token,
                                                            const float* __restrict__ dz_row, float* __restrict__ dcent) {
  const int nc = cdiv(d, 256);
  const int e = blockIdx.x / nc, c = (blockIdx.x % nc) * 256 + threadIdx.x;
  if (e >= N || c >= d) return;
  const int lo = clampi(off[e], 0, n_rows), hi = clampi(off[e + 1], lo, n_rows);
  auto term = [&](int r) -> float {
    const int t = perm_token[r];
    if (t < 0 || t >= T) return 0.0f;
    const size_t o = static_cast<size_t>(t) * d + c;
    const float uv = act_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(u)[o]) : static_cast<const float*>(u)[o];
    return dz_row[r] * uv;
  };
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int r = lo;
  for (; r + 4 <= hi; r += 4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = term(r + j);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += v[j];
  }
  for (int j = 0; r < hi; ++r, ++j) acc[j] += term(r);
  dcent[static_cast<size_t>(e) * d + c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Elementwise over [n_rows, I], 8 consecutive columns per thread (16-byte loads and stores):
// dGU = [dh U SiLU'(G) | dh SiLU(G)] and h = SiLU(G) U.
__global__ __launch_bounds__(256) void swiglu_backward_kernel(long long n8, int I, const uint16_t* __restrict__ dh,
                                                              const uint16_t* __restrict__ gu,
                                                              uint16_t* __restrict__ dgu, uint16_t* __restrict__ h) {
  const int I8 = I / 8;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n8;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long r = i / I8;
    const int c = static_cast<int>(i - r * I8) * 8;
    float g[8], up[8], dv[8], dg[8], du[8], hv[8];
    unpack8(*reinterpret_cast<const uint4*>(gu + r * 2 * I + c), g);
    unpack8(*reinterpret_cast<const uint4*>(gu + r * 2 * I + I + c), up);
    unpack8(*reinterpret_cast<const uint4*>(dh + r * I + c), dv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sg = 1.0f / (1.0f + __expf(-g[k]));
      const float si = g[k] * sg;
      dg[k] = dv[k] * up[k] * sg * (1.0f + g[k] * (1.0f - sg));
      du[k] = dv[k] * si;
      hv[k] = si * up[k];
    }
    store8(dgu + r * 2 * I + c, dg);
    store8(dgu + r * 2 * I + I + c, du);
    store8(h + r * I + c, hv);
  }
}

// du[t] = d_out[t] + du_router[t] + sum_k da[row_of(t, k)] + sum_s da[T K + s T + t], fp32; a block per token,
// 8 consecutive columns per thread (16-byte loads of the bf16 rows).
__device__ __forceinline__ void add_bf16x8(float (&a)[8], const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[2 * i] += __uint_as_float(w[i] << 16);
    a[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(256) void input_grad_kernel(int T, int d, int K, int Ns, const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ du_router,
                                                         const uint16_t* __restrict__ da,
                                                         const int32_t* __restrict__ row_of, int n_rows,
                                                         float* __restrict__ du) {
  const int t = blockIdx.x;
  if (t >= T) return;
  for (int c = 8 * threadIdx.x; c < d; c += 8 * blockDim.x) {
    const size_t o = static_cast<size_t>(t) * d + c;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    add_bf16x8(acc, dout + o);
    if (du_router) {
      const float4 a = reinterpret_cast<const float4*>(du_router + o)[0], b = reinterpret_cast<const float4*>(du_router + o)[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w; acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    for (int k = 0; k < K; ++k) {
      const int r = row_of[static_cast<size_t>(t) * K + k];
      if (r >= 0 && r < n_rows) add_bf16x8(acc, da + static_cast<size_t>(r) * d + c);
    }
    for (int s = 0; s < Ns; ++s) add_bf16x8(acc, da + (static_cast<size_t>(T) * K + static_cast<size_t>(s) * T + t) * d + c);
    reinterpret_cast<float4*>(du + o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(du + o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// W [n][R][C] -> the tiled layout of W^T [n][C][R] (plain 256-row tiles of the
// transposed matrix; rows of W^T past C are zero). A block per (matrix, tile of
// 256 W columns, 32 W rows = one 64-byte K step of W^T): the 32 x 256 piece of W
// goes through LDS and comes out as the step's 16 KB block.
__global__ __launch_bounds__(256) void transpose_tile_kernel(int R, int C, const uint16_t* __restrict__ w,
                                                             uint8_t* __restrict__ out) {
  __shared__ uint16_t sm[32][256 + 2];
  const int ntiles = cdiv(C, 256), nst = R / 32;
  long long b = blockIdx.x;
  const int st = static_cast<int>(b % nst);
  b /= nst;
  const int t = static_cast<int>(b % ntiles);
  const long long mat = b / ntiles;
  const int tid = threadIdx.x;
  for (int i = tid; i < 32 * 256; i += 256) {
    const int rr = i / 256, cc = i % 256;
    const int col = 256 * t + cc;
    sm[rr][cc] = col < C ? w[(static_cast<size_t>(mat) * R + 32 * st + rr) * C + col] : static_cast<uint16_t>(0);
  }
  __syncthreads();
  uint8_t* blk = out + ((static_cast<size_t>(mat) * ntiles + t) * nst + st) * 16384;
  for (int p = tid; p < 1024; p += 256) {               // 16-byte quarters: tile row rw, logical quarter q
    const int rw = p >> 2, q = p & 3;
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = static_cast<uint32_t>(sm[8 * q + 2 * k][rw]) | (static_cast<uint32_t>(sm[8 * q + 2 * k + 1][rw]) << 16);
    *reinterpret_cast<uint4*>(blk + 64 * rw + 16 * (q ^ ((rw >> 2) & 3))) = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

static long long grid_cap(long long blocks) {
  const long long cap = static_cast<long long>(device_cu_count()) * 16;
  return blocks > cap ? cap : (blocks < 1 ? 1 : blocks);
}

hipError_t launch_combine_backward(const Shape& s, const void* dout, const void* y, const int32_t* row_of,
                                   const float* gate, void* dy, bool dy_f32, float* dgate, hipStream_t st) {
  const long long blocks = grid_cap(cdiv(s.T, 4));
  if (dy_f32)
    hipLaunchKernelGGL(combine_backward_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, s.T, s.d,
                       s.K, s.Ns, static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y), row_of, gate,
                       static_cast<float*>(dy), dgate, s.T * s.K);
  else
    hipLaunchKernelGGL(combine_backward_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, s.T,
                       s.d, s.K, s.Ns, static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y), row_of,
                       gate, static_cast<uint16_t*>(dy), dgate, s.T * s.K);
  return hipGetLastError();
}

hipError_t launch_route_backward(const Shape& s, moe_dtype act, const void* u, const void* cent, const float* scores,
                                 const int32_t* idx, const float* dgate, const int32_t* off,
                                 const int32_t* perm_token, const int32_t* row_of, float* du_router, float* dcent,
                                 float* dz_row, hipStream_t st) {
  const int bf = act == MOE_BF16 ? 1 : 0;
  const long long blocks = grid_cap(cdiv(s.T, 4));
  hipLaunchKernelGGL(route_backward_token_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, s.T, s.d, s.N,
                     s.K, bf, cent, scores, idx, dgate, row_of, du_router, dz_row);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(centroid_grad_kernel, dim3(static_cast<unsigned>(s.N * cdiv(s.d, 256))), dim3(256), 0, st, s.T,
                     s.d, s.N, s.T * s.K, bf, u, off, perm_token, dz_row, dcent);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward(long long n_rows, int I, const void* dh, const void* gu, void* dgu, void* h,
                                  hipStream_t st) {
  const long long n8 = n_rows * I / 8;
  const long long blocks = grid_cap((n8 + 255) / 256);
  hipLaunchKernelGGL(swiglu_backward_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, n8, I,
                     static_cast<const uint16_t*>(dh), static_cast<const uint16_t*>(gu), static_cast<uint16_t*>(dgu),
                     static_cast<uint16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_input_grad(const Shape& s, const void* dout, const float* du_router, const void* da,
                             const int32_t* row_of, float* du, hipStream_t st) {
  hipLaunchKernelGGL(input_grad_kernel, dim3(static_cast<unsigned>(s.T)), dim3(256), 0, st, s.T, s.d, s.K, s.Ns,
                     static_cast<const uint16_t*>(dout), du_router, static_cast<const uint16_t*>(da), row_of,
                     s.T * s.K, du);
  return hipGetLastError();
}

hipError_t launch_transpose_tile_bf16(int n_mats, int rows, int cols, const void* w, void* out, hipStream_t st) {
  const long long blocks = static_cast<long long>(n_mats) * cdiv(cols, 256) * (rows / 32);
  hipLaunchKernelGGL(transpose_tile_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, rows, cols,
                     static_cast<const uint16_t*>(w), static_cast<uint8_t*>(out));
  return hipGetLastError();
}

}  // namespace moe
