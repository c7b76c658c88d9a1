// Weight gradients of the grouped expert FFN ("DeepSeek_V3_Report: Annotation",
// FP8 framework: the weight-gradient GEMM of each linear layer, weight
// gradients kept in fp32):
//   C[e][m][n] = sum over the rows r of expert e of X[r][m] * Y[src(r)][n],
// the contraction running over the expert's ragged rows (dW_d = dy^T h,
// dW_gate_up = [dG | dU]^T a). bf16 operands, fp32 MFMA accumulation, fp32
// output; experts without rows get zeros.
//
// Both operands hold the contraction index (the row) as their slow axis, the
// transpose of what an MFMA operand wants (8 consecutive K values per lane).
// The tiles are staged in LDS as they lie in HBM (row-major, 16-byte loads and
// stores) and the transpose happens on the way out of LDS: gfx950's
// ds_read_b64_tr_b16 gives lane i of each 16-lane group element i of the four
// 4-element pieces that lanes 4j .. 4j + 3 point at, so pointing the 16 lanes
// at 4 rows x 16 columns hands every lane 4 consecutive rows of one column.
// Two such reads make one 32x32x16 operand.
//
// A workgroup per (expert, 256 x 256 output tile), eight waves in a 2 x 4 grid
// of 128 x 64 (4 x 2 MFMA tiles of 32 x 32), one workgroup per CU: the tile
// re-reads the X rows once per 256 output columns instead of per 128, so the
// direct-to-LDS traffic per output falls by a third. Rows advance in chunks of
// 32 through a ring of three 32 KB LDS stages filled by direct-to-LDS buffer
// loads (no VGPR staging), two chunks ahead of the one being multiplied. LDS rows are XOR-swizzled in 16-byte slots (slot = column
// chunk ^ 4 (row % 4)) so the 4 rows of one transpose read fall in 4 different
// bank quadrants; a DMA load writes 64 consecutive slots, so each lane fetches
// the global chunk that belongs at its slot. Rows past the expert's last,
// columns past M and unmapped source rows fall outside the loads' buffer range
// and arrive as zeros. Tiles run expert-major with each expert's M tiles spread
// over the XCDs (below); the fp32 tile is written with non-temporal stores (it
// is not read again by this pass).
#include <mutex>

#include "common.h"
#include "gemm_pipe.h"
#include "launch.h"
#include "sched.h"

namespace moe {

namespace {

constexpr int kWgBM = 256, kWgBN = 256, kWgBK = 32, kWgNT = 512;
constexpr int kWgXBytes = kWgBK * kWgBM * 2;              // 16 KB
constexpr int kWgStage = kWgXBytes + kWgBK * kWgBN * 2;   // + 16 KB

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// LDS byte address of this lane's first transpose read of the 32 x 16 (column x
// K) operand at column col0 of a row-major LDS tile of pitch `pitch` bytes at
// LDS address `tile` (rows k0 = 0): lane l gets column col0 + l % 32, rows
// 8 (l / 32) .. + 3 from this read and + 4 .. + 7 from the one 4 rows further.
__device__ __forceinline__ uint32_t tr_addr(uint32_t tile, int pitch, int col0) {
  const int l = threadIdx.x & 63, g = l >> 4, p = l & 15, j = p >> 2, q = p & 3;
  const int col = col0 + 16 * (g & 1) + 4 * q;               // start of this lane's 4-column piece
  const int k = 8 * (g >> 1) + j;                             // k % 4 == j
  return tile + k * pitch + (((col >> 3) ^ (4 * j)) << 4) + ((col & 7) << 1);
}

// The twelve transpose reads of one K16 step (rows ks .. ks + 15 of the stage):
// four X operands at xa[0..3], two Y operands at ya[0..1]. The reads are waited
// for inside the same statement, so every output is complete when it returns.
template <int KS>
__device__ __forceinline__ void tr_step(i32x2 (&r)[12], const uint32_t (&xa)[4], const uint32_t (&ya)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12 offset:%18\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:%19\n\t"
      "ds_read_b64_tr_b16 %2, %13 offset:%18\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:%19\n\t"
      "ds_read_b64_tr_b16 %4, %14 offset:%18\n\t"
      "ds_read_b64_tr_b16 %5, %14 offset:%19\n\t"
      "ds_read_b64_tr_b16 %6, %15 offset:%18\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%19\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:%21\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
      : "v"(xa[0]), "v"(xa[1]), "v"(xa[2]), "v"(xa[3]), "v"(ya[0]), "v"(ya[1]), "n"(KS * kWgBM * 2),
        "n"((KS + 4) * kWgBM * 2), "n"(KS * kWgBN * 2), "n"((KS + 4) * kWgBN * 2));
}

__device__ __forceinline__ bf16x8 tr_pair(const i32x2& lo, const i32x2& hi) {
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6,
                                 7);
}

}  // namespace

namespace {

constexpr int kWgNS = 3;                                  // ring stages
constexpr uint32_t kWgOut = 0xFFFFFFF0u;                  // a voffset past every buffer range: loads zero
constexpr uint64_t kWgMaxRange = 0xFFFFFF00ull;

__device__ __forceinline__ uint32_t range_bytes(long long bytes) {
  return static_cast<uint32_t>(bytes <= 0 ? 0 : (bytes > static_cast<long long>(kWgMaxRange) ? kWgMaxRange : bytes));
}

template <int N>
__device__ __forceinline__ void wg_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace

// GATHER: the Y rows come through row_src (read with scalar loads when the
// chunk's DMA is issued: four rows per wave and load, picked per lane), so the
// vector-memory counter only ever counts the DMA loads; otherwise Y row r is r
// (direct) or r - lo (segment).
template <bool GATHER>
__global__ __launch_bounds__(kWgNT, 1) void wgrad_kernel(int M, int N, int E, int n_rows, int a_rows,
                                                       const int32_t* __restrict__ off, moe_row_mode mode,
                                                       const int32_t* __restrict__ row_src,
                                                       const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y,
                                                       float* __restrict__ C) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int mt = cdiv(M, kWgBM), nt = cdiv(N, kWgBN);
  // XCD-aware tiles: workgroups go to the 8 XCDs round-robin, and XCD x takes the M tiles mi of expert e with
  // (mi + e) % 8 == x, each with all its N tiles, in expert order: an expert's X rows are fetched once (each M
  // tile by one XCD), its Y rows once per XCD, and all XCDs work on the same experts at a time. (Measured at
  // the V3 shape: 4.87 -> 4.83 ms for dW_down, whose X fetch drops from 8.8 to 3.5 GB, and 8.6 -> 8.45 ms for
  // dW_gate_up; splitting the N tiles of its larger Y instead fetched less but took 8.9 ms.)
  const int x = static_cast<int>(blockIdx.x & 7);
  const long long slot = blockIdx.x >> 3;
  const long long per8 = static_cast<long long>(mt) * nt;    // tiles of XCD x over 8 consecutive experts
  int e = static_cast<int>(slot / per8) * 8;
  int rem = static_cast<int>(slot % per8), mfirst = 0;
  for (int r = 0; r < 8; ++r) {                              // expert e + r: M tiles mfirst, mfirst + 8, ...
    mfirst = (x - (e + r) % 8 + 8) % 8;
    const int cnt = (mfirst < mt ? (mt - mfirst + 7) / 8 : 0) * nt;
    if (rem < cnt) {
      e += r;
      break;
    }
    rem -= cnt;
  }
  if (e >= E) return;
  const int m0 = (mfirst + 8 * (rem / nt)) * kWgBM, n0 = (rem % nt) * kWgBN;
  const int lo = clampi(off[e], 0, n_rows), hi = clampi(off[e + 1], lo, n_rows);
  const int tid = threadIdx.x, l = tid & 63, wm = (tid >> 6) >> 2, wn = (tid >> 6) & 3;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // M or N % 256 == 128: the last tile's second half (in that dimension) is empty
  const bool active = m0 + wm * 128 < M && n0 + wn * 64 < N;
  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
  const int nch = cdiv(hi - lo, kWgBK);
  const uint32_t lds_addr =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)lds));
  uint32_t xo[4], yo[2];                                      // transpose-read offsets within a stage
#pragma unroll
  for (int a = 0; a < 4; ++a) xo[a] = tr_addr(0, kWgBM * 2, wm * 128 + a * 32);
#pragma unroll
  for (int c = 0; c < 2; ++c) yo[c] = tr_addr(kWgXBytes, kWgBN * 2, wn * 64 + c * 32);
  auto mma_step = [&](const i32x2 (&r)[12], f32x16 (&ac)[4][2]) {
    bf16x8 fb[2] = {tr_pair(r[8], r[9]), tr_pair(r[10], r[11])};
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const bf16x8 fa = tr_pair(r[2 * a], r[2 * a + 1]);
#pragma unroll
      for (int c = 0; c < 2; ++c) ac[a][c] = mfma_32x32x16_bf16(fa, fb[c], ac[a][c]);
    }
  };

  if (nch > 0) {
    // DMA load q of this wave fills LDS slots (q * 8 + w) * 64 + lane of the X (or Y) part of a stage: two
    // 512-byte rows, the lanes of each at the 16-byte slots of their row
    uint32_t vx[2], vy[2];
    int yrow[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 2 * (q * 8 + w) + (l >> 5), c = (l & 31) ^ (4 * (row & 3));
      vx[q] = static_cast<uint32_t>(row * M * 2 + c * 16);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      yrow[q] = 2 * (q * 8 + w) + (l >> 5);
      const int c = (l & 31) ^ (4 * (yrow[q] & 3));
      vy[q] = static_cast<uint32_t>(GATHER ? c * 16 : yrow[q] * N * 2 + c * 16);
    }
    auto issue = [&](int ch) {
      const int r0 = lo + kWgBK * ch;
      uint8_t* st = lds + (ch % kWgNS) * kWgStage;
      const __amdgpu_buffer_rsrc_t rx =
          pipe_rsrc(X + static_cast<size_t>(r0) * M + m0, range_bytes((static_cast<long long>(hi - r0) * M - m0) * 2));
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(st + (q * 8 + w) * 1024), 16, vx[q], 0, 0, 0);
      if (GATHER) {
        const __amdgpu_buffer_rsrc_t ry =
            pipe_rsrc(Y + n0, range_bytes((static_cast<long long>(a_rows) * N - n0) * 2));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int base = r0 + 2 * (q * 8 + w);                 // wave-uniform: scalar loads, clamped to the rows
          const int s0 = row_src[min(base, hi - 1)], s1 = row_src[min(base + 1, hi - 1)];
          const int sr = (l >> 5) ? s1 : s0;
          const bool ok = r0 + yrow[q] < hi && sr >= 0 && sr < a_rows;
          const uint32_t vo = ok ? static_cast<uint32_t>(sr) * static_cast<uint32_t>(N * 2) + vy[q] : kWgOut;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void_t*)(st + kWgXBytes + (q * 8 + w) * 1024), 16, vo, 0,
                                                   0, 0);
        }
      } else {
        const int s0 = mode == MOE_ROWS_SEGMENT ? r0 - lo : r0;
        const int yrows = min(hi - r0, a_rows - s0);
        const __amdgpu_buffer_rsrc_t ry = pipe_rsrc(
            Y + static_cast<size_t>(s0) * N + n0, yrows > 0 ? range_bytes((static_cast<long long>(yrows) * N - n0) * 2)
                                                            : 0u);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void_t*)(st + kWgXBytes + (q * 8 + w) * 1024), 16, vy[q],
                                                   0, 0, 0);
      }
    };
    // prologue: chunks 0 and 1 in flight
    issue(0);
    if (nch > 1) issue(1);
    // iteration ch: wait for chunk ch (only chunk ch + 1's four loads may still be in flight), issue the DMA of
    // chunk ch + 2 into the stage chunk ch - 1 used, multiply chunk ch
    for (int ch = 0; ch < nch; ++ch) {
      if (ch + 1 < nch) wg_wait_barrier<4>();
      else wg_wait_barrier<0>();
      if (ch + 2 < nch) issue(ch + 2);
      if (active) {
        const uint32_t st = lds_addr + (ch % kWgNS) * kWgStage;
        const uint32_t xa[4] = {st + xo[0], st + xo[1], st + xo[2], st + xo[3]};
        const uint32_t ya[2] = {st + yo[0], st + yo[1]};
        i32x2 r[12];
        tr_step<0>(r, xa, ya);
        mma_step(r, acc);
        tr_step<16>(r, xa, ya);
        mma_step(r, acc);
      }
    }
  }
  if (!active) return;
  float* Ce = C + static_cast<size_t>(e) * M * N;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int n = n0 + wn * 64 + c * 32 + (l & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 128 + a * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        __builtin_nontemporal_store(acc[a][c][v], Ce + static_cast<size_t>(m) * N + n);
      }
    }
}

hipError_t launch_wgrad(int M, int N, int E, int n_rows, int a_rows, const int32_t* off, moe_row_mode mode,
                        const int32_t* row_src, const void* X, const void* Y, float* C, hipStream_t st) {
  static std::once_flag once;
  std::call_once(once, [] {
    for (const void* k : {reinterpret_cast<const void*>(wgrad_kernel<true>),
                          reinterpret_cast<const void*>(wgrad_kernel<false>)})
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kWgNS * kWgStage);
    (void)hipGetLastError();
  });
  const long long blocks = 8LL * ((E + 7) / 8) * cdiv(M, kWgBM) * cdiv(N, kWgBN);   // whole groups of 8 experts
  const size_t lds = static_cast<size_t>(kWgNS) * kWgStage;
  if (mode == MOE_ROWS_GATHER)
    hipLaunchKernelGGL(wgrad_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kWgNT), lds, st, M, N, E, n_rows,
                       a_rows, off, mode, row_src, static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Y), C);
  else
    hipLaunchKernelGGL(wgrad_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kWgNT), lds, st, M, N, E, n_rows,
                       a_rows, off, mode, row_src, static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Y), C);
  return hipGetLastError();
}

}  // namespace moe
