// Internal host-side launchers; the C ABI in api.hip validates arguments and
// then calls these. Every launcher only enqueues work on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

struct Shape {
  int T, d, N, G, M, topn, K, Ns, I;
  int bi;   // batch-invariant mode
};

inline Shape to_shape(const moe_shape& s) {
  return Shape{s.T, s.d, s.n_routed, s.n_groups, s.topk_groups, s.group_topn, s.topk, s.n_shared, s.inter,
               s.batch_invariant};
}

// Compute units of the current device (cached per device).
int device_cu_count();

// Zero the kQueueInts counters of a grouped FFN launch's unit queue
// (sched.h) on st, with a kernel (graph-capture safe).
hipError_t launch_queue_reset(int* q, hipStream_t st);

// ---- route
// workspace: the scores [T, N] fp32 (used when the caller passes none), then
// for bf16 the partial logit sums of the K slices.
size_t route_ws_bytes(const Shape& s, moe_dtype act);
hipError_t launch_route(const Shape& s, moe_dtype act, const void* u, const void* cent, const float* bias,
                        int32_t* idx, float* gate, int32_t* load, float* scores, void* ws, hipStream_t st);

// ---- permute
size_t permute_ws_bytes(const Shape& s);
hipError_t launch_permute_maps(const Shape& s, const int32_t* idx, int32_t* offsets, int32_t* perm,
                               int32_t* row_of, void* ws, hipStream_t st);
// rows r < n_rows of dst = src[index[r]] (index may be null: identity); dst in
// dst_dtype (same as src, or E4M3 with 1x128 scales).
hipError_t launch_rows_copy(int n_rows, int d, moe_dtype src_dtype, const void* src, int src_rows,
                            const int32_t* index, moe_dtype dst_dtype, void* dst, float* dst_scale,
                            hipStream_t st);

// ---- balance statistics (eq. (17)-(20))
size_t balance_ws_bytes(const Shape& s, int seq_len);
hipError_t launch_balance_stats(const Shape& s, const float* scores, const int32_t* idx, int seq_len, float alpha,
                                float* f, float* P, float* loss, void* ws, hipStream_t st);

// ---- combine / bias
hipError_t launch_combine(const Shape& s, moe_dtype io, const void* u, const void* y, const int32_t* row_of,
                          const float* gate, const void* ysh, void* out, hipStream_t st);
hipError_t launch_bias_update(const Shape& s, const int32_t* load, float gamma, float* bias, hipStream_t st);

// ---- expert FFN
struct FfnArgs {
  int d, I, n_experts, n_rows, a_rows;
  const int32_t* offsets;
  moe_row_mode mode;
  const int32_t* row_src;
  const void* a;
  const float* a_scale;
  const void* w_gu;
  const void* w_gu_scale;   // fp32 per 128x128 block (E4M3 weights) or E8M0 bytes (MXFP4)
  const void* w_d;
  const void* w_d_scale;
  moe_dtype y_dtype;
  void* y;
  void* h;         // SwiGLU output [n_rows, I]
  float* h_scale;  // fp8: [n_rows, I/128]
  int* queue;      // unit-queue counters of this launch (kQueueInts ints of workspace)
  void* gu_cache = nullptr;   // the SwiGLU inputs [n_rows, 2I] for the backward (bf16, or E4M3 codes), or NULL
  float* gu_scale = nullptr;  // fp8: the cache's 1x128 scales [n_rows, 2I / 128]
};
constexpr size_t kFfnQueueBytes = 128;   // per launch
// Workspace of moe_grouped_ffn: H (+ its fp8 scales), then the queue
// counters of the gate/up and the down launch at ffn_queue_offset.
size_t ffn_queue_offset(moe_dtype w, int n_rows, int I);
size_t ffn_ws_bytes(moe_dtype w, int n_rows, int I);
hipError_t launch_ffn_f32_gate_up(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_f32_down(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_bf16_gate_up(const FfnArgs& a, hipStream_t st, bool tiled);
hipError_t launch_ffn_bf16_down(const FfnArgs& a, hipStream_t st, bool tiled);
hipError_t launch_ffn_fp8_gate_up(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_fp8_down(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_fp4_gate_up(const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_fp4_down(const FfnArgs& a, hipStream_t st);

// ---- backward
hipError_t launch_combine_backward(const Shape& s, const void* dout, const void* y, const int32_t* row_of,
                                   const float* gate, void* dy, bool dy_f32, float* dgate, hipStream_t st);
hipError_t launch_route_backward(const Shape& s, moe_dtype act, const void* u, const void* cent, const float* scores,
                                 const int32_t* idx, const float* dgate, const int32_t* off,
                                 const int32_t* perm_token, const int32_t* row_of, float* du_router, float* dcent,
                                 float* dz_row, hipStream_t st);
hipError_t launch_swiglu_backward(long long n_rows, int I, const void* dh, const void* gu, void* dgu, void* h,
                                  hipStream_t st);
hipError_t launch_input_grad(const Shape& s, const void* dout, const float* du_router, const void* da,
                             const int32_t* row_of, float* du, hipStream_t st);
hipError_t launch_transpose_tile_bf16(int n_mats, int rows, int cols, const void* w, void* out, hipStream_t st);
// FP8 backward (backward_fp8.hip)
hipError_t launch_transpose_rows_bf16(int n_mats, int rows, int cols, const void* w, void* out, hipStream_t st);
hipError_t launch_quantize_rows(long long n_rows, int cols, const void* x, bool f32_in, void* codes, float* scales,
                                hipStream_t st);
hipError_t launch_swiglu_backward8(long long n_rows, int I, const void* dh, const void* guq, const float* gus,
                                   void* dgu, void* h, hipStream_t st);
hipError_t launch_row_block_prefix(int E, int n_rows, const int32_t* off, int* pre, hipStream_t st);
hipError_t launch_requant_cols(int C, int E, int n_rows, const int32_t* off, const int* pre, moe_row_mode mode,
                               const int32_t* row_src, int a_rows, const void* x, bool f32_in, const void* xq,
                               const float* xs, void* out, hipStream_t st);
hipError_t launch_wgrad(int M, int N, int E, int n_rows, int a_rows, const int32_t* off, moe_row_mode mode,
                        const int32_t* row_src, const void* X, const void* Y, float* C, hipStream_t st);

// ---- weight preparation
hipError_t launch_quantize_weights(int n_mats, int rows, int cols, int gate_up, const void* w, void* codes,
                                   float* scale, hipStream_t st);
hipError_t launch_tile_weights_bf16(int n_mats, int rows, int cols, int gate_up, const void* src, void* dst,
                                    hipStream_t st);
hipError_t launch_quantize_weights_mxfp4(int n_mats, int rows, int cols, int gate_up, const void* w, void* codes,
                                         void* scales, hipStream_t st);

}  // namespace moe
