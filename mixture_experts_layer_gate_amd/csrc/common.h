// Shared device helpers of the gfx950 MoE kernels: vector types, MFMA
// wrappers, bf16 / E4M3 conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------- E4M3 (OCP E4M3FN)
// Saturating round-to-nearest-even encode of an fp32 value: |x| >= 448 maps to
// +-448 (code 0x7E), values below 2^-6 land on the subnormal grid m * 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = __builtin_fabsf(x);
  if (!(a < kE4M3Max)) return sign | ((a != a) ? 0x7Fu : 0x7Eu);
  if (a < 0.015625f) {                         // subnormal: step 2^-9
    const float m = a * 512.0f;                // exact
    return sign | static_cast<uint32_t>(__builtin_rintf(m));   // 8 -> code 0x08 = 2^-6
  }
  const int e = static_cast<int>((b >> 23) & 0xFFu) - 127;     // -6 .. 8
  const uint32_t mant = b & 0x7FFFFFu;
  uint32_t q = mant >> 20;
  const uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;    // q == 8 carries into the exponent
  return sign | ((static_cast<uint32_t>(e + 7) << 3) + q);
}

// Four fp32 values to E4M3 codes packed little-endian (byte r = value r), by
// gfx950's v_cvt_pk_fp8_f32 (round to nearest even) after a clamp to +-448
// that supplies the saturation; NaN stays NaN. Same codes as f32_to_e4m3 for
// every non-NaN input: checked on the GPU over every fp32 value of magnitude
// <= 448, and the clamp maps larger ones to the saturated code.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  auto sat = [](float x) { return x != x ? x : fminf(fmaxf(x, -kE4M3Max), kE4M3Max); };
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), lo, true);
}

// ---------------------------------------------------------------- MFMA
// 32x32x16 bf16 -> fp32. Operand lane layout: lane l supplies row/column
// (l % 32) and the 8 consecutive K values starting at 8 * (l / 32).
// Accumulator layout: element v of lane l is (row 8*(v/4) + 4*(l/32) + v%4, col l%32).
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 fp8(E4M3) x fp8(E4M3) -> fp32, unit block scales. Lane l supplies
// row/column (l % 16) and 32 K bytes of K group (l / 16). Accumulator element
// v of lane l is (row 4*(l/16) + v, col l%16).
__device__ __forceinline__ f32x4 mfma_16x16x128_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------- misc

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace moe
