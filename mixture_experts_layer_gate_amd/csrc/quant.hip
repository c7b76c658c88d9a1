// 128x128 block quantisation of bf16 expert weights to E4M3 with one fp32
// scale per block ("DeepSeek_V3_Report: Annotation", section "Fine-Grained
// Quantization"; scale from the block's max-abs, section "Online Quantization"),
// and the MXFP4 quantisation; both write the codes in the tiled layouts the
// grouped FFN kernels stream.
#include "common.h"
#include "launch.h"

namespace moe {

// Tiled code layout (the E4M3 grouped FFN streams it; see moe_quantize_weights):
// tiles of 256 rows, tile row rw of tile t being matrix row 256 t + rw, or for
// gate_up the gate / up row of the tile's 128 H columns that the tile's waves
// pair; per 64-wide K step a tile's 64-byte row pieces form one 16 KB block,
// row rw at 64 rw with its 16-byte quarter c at 16 (c ^ ((rw >> 2) & 3)).
__device__ __forceinline__ int tiled_row(int t, int rw, int gate_up, int half) {
  if (!gate_up) return 256 * t + rw;
  const int j = (rw >> 5) & 3;
  const int hc = 128 * t + 64 * (rw >> 7) + 32 * (j & 1) + (rw & 31);
  return j >= 2 ? half + hc : hc;
}

// One block of 256 threads per 128x128 weight block; thread t covers row t/2,
// columns 64*(t%2) .. +63. Codes go to the tiled layout, scales to
// [mat][rows/128][cols/128].
__global__ __launch_bounds__(256) void quantize_blocks_kernel(int rows, int cols, int gate_up,
                                                              const uint16_t* __restrict__ w,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float wmax[4];
  const int bc = cols / 128, br = rows / 128, ntiles = (rows + 255) / 256;
  const long long blk = blockIdx.x;
  const long long mat = blk / (static_cast<long long>(br) * bc);
  const int rem = static_cast<int>(blk % (static_cast<long long>(br) * bc));
  const int bi = rem / bc, bj = rem % bc;
  const int r = bi * 128 + (threadIdx.x >> 1);
  const int c0 = bj * 128 + (threadIdx.x & 1) * 64;
  const size_t base = (static_cast<size_t>(mat) * rows + r) * cols + c0;
  float x[64];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint4 p = *reinterpret_cast<const uint4*>(w + base + 8 * v);
    const uint32_t ww[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * v + 2 * i] = __uint_as_float(ww[i] << 16);
      x[8 * v + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, __builtin_fabsf(x[i]));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
  // tile position of matrix row r (the inverse of tiled_row)
  int t, rw;
  if (gate_up) {
    const int half = rows / 2, up = r >= half, hc = up ? r - half : r;
    t = hc / 128;
    const int hl = hc % 128;                        // H column within the tile
    rw = 128 * (hl >> 6) + 32 * ((up ? 2 : 0) + ((hl >> 5) & 1)) + (hl & 31);
  } else {
    t = r / 256;
    rw = r % 256;
  }
  const size_t tile = static_cast<size_t>(mat) * ntiles + t;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* xi = x + 16 * v + 4 * i;
      o[i] = f32x4_to_e4m3(xi[0] * inv, xi[1] * inv, xi[2] * inv, xi[3] * inv);
    }
    const int k = c0 + 16 * v;                      // first K index of this 16-byte piece
    const size_t off = (tile * (cols / 64) + k / 64) * 16384 + 64 * rw + 16 * (((k % 64) / 16) ^ ((rw >> 2) & 3));
    *reinterpret_cast<uint4*>(q + off) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (threadIdx.x == 0)
    scale[(static_cast<size_t>(mat) * br + bi) * bc + bj] = amax > 0.0f ? amax / kE4M3Max : 1.0f;
}

// Zero codes of the padding rows of the last tile (rows % 256 == 128, not gate_up).
__global__ __launch_bounds__(256) void zero_tile_padding_kernel(long long n, int rows, int cols, uint8_t* __restrict__ q) {
  const int ntiles = (rows + 255) / 256, nst = cols / 64;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    // i enumerates (mat, stage, padding row rw in 128..255, 16-byte quarter)
    const int quarter = static_cast<int>(i & 3);
    const int rw = 128 + static_cast<int>((i >> 2) & 127);
    const long long ms = i >> 9;
    const int st = static_cast<int>(ms % nst);
    const long long mat = ms / nst;
    const size_t off = ((static_cast<size_t>(mat) * ntiles + ntiles - 1) * nst + st) * 16384 + 64 * rw + 16 * quarter;
    *reinterpret_cast<uint4*>(q + off) = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_quantize_weights(int n_mats, int rows, int cols, int gate_up, const void* w, void* codes,
                                   float* scale, hipStream_t st) {
  const long long blocks = static_cast<long long>(n_mats) * (rows / 128) * (cols / 128);
  hipLaunchKernelGGL(quantize_blocks_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, rows, cols, gate_up,
                     static_cast<const uint16_t*>(w), static_cast<uint8_t*>(codes), scale);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (rows % 256 != 0) {
    const long long n = static_cast<long long>(n_mats) * (cols / 64) * 128 * 4;
    long long b = (n + 255) / 256;
    const long long cap = static_cast<long long>(device_cu_count()) * 32;
    if (b > cap) b = cap;
    hipLaunchKernelGGL(zero_tile_padding_kernel, dim3(static_cast<unsigned>(b)), dim3(256), 0, st, n, rows, cols,
                       static_cast<uint8_t*>(codes));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- bf16 tiles
// Rows of row_bytes bytes (a multiple of 64) rearranged into the tiled layout
// with 64-byte K steps (moe_tile_weights_bf16): a thread per 16-byte quarter,
// quarters fastest, then tile rows, so a wave reads 16 rows' 64-byte pieces.
__global__ __launch_bounds__(256) void tile_rows_kernel(long long n, int rows, int row_bytes, int gate_up,
                                                        const uint8_t* __restrict__ src, uint8_t* __restrict__ dst) {
  const int ntiles = (rows + 255) / 256, nst = row_bytes / 64, half = rows / 2;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(i & 3), rw = static_cast<int>((i >> 2) & 255);
    long long rest = i >> 10;
    const int st = static_cast<int>(rest % nst);
    rest /= nst;
    const int t = static_cast<int>(rest % ntiles);
    const long long mat = rest / ntiles;
    const int row = tiled_row(t, rw, gate_up, half);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < rows) v = *reinterpret_cast<const uint4*>(src + (static_cast<size_t>(mat) * rows + row) * row_bytes + st * 64 + 16 * c);
    const size_t off = ((static_cast<size_t>(mat) * ntiles + t) * nst + st) * 16384 + 64 * rw + 16 * (c ^ ((rw >> 2) & 3));
    *reinterpret_cast<uint4*>(dst + off) = v;
  }
}

hipError_t launch_tile_weights_bf16(int n_mats, int rows, int cols, int gate_up, const void* src, void* dst,
                                    hipStream_t st) {
  const long long n = static_cast<long long>(n_mats) * ((rows + 255) / 256) * (cols * 2 / 64) * 1024;
  long long blocks = (n + 255) / 256;
  const long long cap = static_cast<long long>(device_cu_count()) * 32;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(tile_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, n, rows, cols * 2, gate_up,
                     static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

// ---------------------------------------------------------------- MXFP4
// OCP microscaling FP4 of bf16 weights along each row ("DeepSeek V3 / V4
// Infra", V4 post-training FP4 QAT of the expert weights): per 32 consecutive
// values of a row, k = floor(log2(amax)) - 2 (at least -127; 0 for an
// all-zero block), E8M0 scale byte k + 127, and E2M1 codes of x * 2^-k, round
// to nearest with ties to the even code, saturating at 6, sign from x.

// E2M1 code of y: count the decision points below |y| (a tie goes to the even
// code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fminf(__builtin_fabsf(y), 6.0f);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(y) >> 31) << 3);
}

// One thread per (tile row, 32-value block); a wave covers 64 consecutive tile
// rows of one K block, so its scale bytes are one contiguous run. Output in
// the tiled layout the MXFP4 grouped FFN streams (see moe_quantize_weights_mxfp4):
// tile row rw of tile t is matrix row 256 t + rw, or for gate_up the gate / up
// row of the tile's 128 H columns that the tile's waves pair; rows past the
// matrix are zero.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(long long n_blocks, int rows, int cols, int gate_up,
                                                             const uint16_t* __restrict__ w,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int kbs = cols / 32, ntiles = cdiv(rows, 256), half = rows / 2;
  for (long long b = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; b < n_blocks;
       b += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int rw = static_cast<int>(b & 255);
    long long rest = b >> 8;
    const int kb = static_cast<int>(rest % kbs);
    rest /= kbs;
    const int t = static_cast<int>(rest % ntiles);
    const long long mat = rest / ntiles;
    const int row = tiled_row(t, rw, gate_up, half);
    float x[32];
    if (row < rows) {
      const uint16_t* src = w + (static_cast<size_t>(mat) * rows + row) * cols + static_cast<size_t>(kb) * 32;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 p = *reinterpret_cast<const uint4*>(src + 8 * v);
        const uint32_t ww[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[8 * v + 2 * i] = __uint_as_float(ww[i] << 16);
          x[8 * v + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, __builtin_fabsf(x[i]));
    int k = 0;
    if (amax > 0.0f) {
      int e;
      (void)__builtin_frexpf(amax, &e);   // amax = m 2^e, 0.5 <= m < 1: floor(log2 amax) = e - 1
      k = max(e - 3, -127);
    }
    uint32_t o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= e2m1_code(__builtin_ldexpf(x[8 * v + i], -k)) << (4 * i);
      o[v] = word;
    }
    const size_t tile = static_cast<size_t>(mat) * ntiles + t;
    const size_t coff = (tile * (cols / 64) + (kb >> 1)) * 8192 + 32 * rw + 16 * ((kb & 1) ^ ((rw >> 3) & 1));
    *reinterpret_cast<uint4*>(codes + coff) = make_uint4(o[0], o[1], o[2], o[3]);
    scales[(tile * (cols / 128) + (kb >> 2)) * 1024 + (kb & 3) * 256 + rw] = static_cast<uint8_t>(k + 127);
  }
}

hipError_t launch_quantize_weights_mxfp4(int n_mats, int rows, int cols, int gate_up, const void* w, void* codes,
                                         void* scales, hipStream_t st) {
  const long long n = static_cast<long long>(n_mats) * cdiv(rows, 256) * 256 * (cols / 32);
  long long blocks = (n + 255) / 256;
  const long long cap = static_cast<long long>(device_cu_count()) * 32;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, n, rows, cols,
                     gate_up, static_cast<const uint16_t*>(w), static_cast<uint8_t*>(codes),
                     static_cast<uint8_t*>(scales));
  return hipGetLastError();
}

}  // namespace moe
