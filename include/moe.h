/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer forward.
 *
 * The layer is the DeepSeekMoE FFN of the DeepSeek-V3 report ("DeepSeek_V3_Report:
 * Annotation", section "DeepSeekMoE with Auxiliary-Loss-Free Load Balancing",
 * eq. (12)-(16)): sigmoid affinities, an expert bias used only to select the
 * top-K experts inside the M best expert groups, gates normalised over the
 * selected raw affinities, SwiGLU experts, a gate-weighted combine with the
 * shared experts and the residual, and the step-end bias update.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless stated; arrays are dense and
 *    row-major. The caller owns every buffer; the library never allocates,
 *    frees or keeps a pointer after a call returns. Scratch memory comes in
 *    through `workspace` (size from moe_workspace_bytes).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Each
 *    call only enqueues work on it and returns; no call synchronises the host,
 *    except when the environment variable MOE_SYNC_DEBUG=1 is set (then every
 *    call waits for its stream and reports kernel errors).
 *  - Arguments are validated on the host before anything is launched:
 *    MOE_E_INVALID for a null required pointer, a non-positive size or an
 *    inconsistent shape; MOE_E_UNSUPPORTED for shapes or dtypes the library
 *    does not handle; MOE_E_WORKSPACE when ws_bytes is too small; MOE_E_HIP
 *    when a launch fails. The message of the last non-OK status of the calling
 *    thread is returned by moe_last_error(). No exception crosses the ABI.
 *  - Device-side integer inputs (expert ids, offsets, row indices) are range
 *    checked by the kernels: an out-of-range entry is never dereferenced; it
 *    is skipped, or the output rows that depend on it hold unspecified values.
 *  - Calls are re-entrant; calls on different streams may run concurrently
 *    if they do not share output or workspace buffers.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_INVALID = 1,
  MOE_E_UNSUPPORTED = 2,
  MOE_E_WORKSPACE = 3,
  MOE_E_HIP = 4
} moe_status;

typedef enum {
  MOE_F32 = 0,     /* IEEE binary32 */
  MOE_BF16 = 1,    /* bfloat16 */
  MOE_F8E4M3 = 2,  /* OCP E4M3FN: bias 7, max 448, no infinities */
  MOE_F8E4M3_POW2 = 3, /* E4M3FN codes with power-of-two tile scales (an a_dtype of moe_permute only) */
  MOE_F4E2M1 = 4,     /* OCP MXFP4 weights (a weight dtype only): E2M1 codes, two per byte with the
                         even K index in the low nibble, one E8M0 scale byte (2^(b - 127)) per 32
                         consecutive K values, in the tiled layout of moe_quantize_weights_mxfp4 */
  MOE_BF16_TILED = 5  /* bf16 weights in the tiled layout of moe_tile_weights_bf16 (a weight dtype
                         only; activations, H and y as with MOE_BF16) */
} moe_dtype;

/* How moe_grouped_ffn finds the input row of output row r of expert e. */
typedef enum {
  MOE_ROWS_DIRECT = 0,   /* a[r]                       (a already permuted)      */
  MOE_ROWS_GATHER = 1,   /* a[row_src[r]]              (gather fused in the GEMM) */
  MOE_ROWS_SEGMENT = 2   /* a[r - expert_offsets[e]]   (shared experts: all tokens) */
} moe_row_mode;

/* Host struct. N_r = n_routed experts in n_groups contiguous groups of
 * S = N_r / n_groups; each token keeps the topk_groups (M) groups with the
 * highest group score (sum of the group_topn largest biased affinities of the
 * group) and selects topk (K) experts inside them. */
typedef struct {
  int32_t T;            /* tokens                                  */
  int32_t d;            /* hidden size, multiple of 128            */
  int32_t n_routed;     /* N_r <= 1024                             */
  int32_t n_groups;     /* G, divides N_r, <= 64                   */
  int32_t topk_groups;  /* M <= G                                  */
  int32_t group_topn;   /* 1..4, <= S                              */
  int32_t topk;         /* K <= 16, K <= M * S                     */
  int32_t n_shared;     /* N_s >= 0                                */
  int32_t inter;        /* I, SwiGLU width, multiple of 128        */
  int32_t batch_invariant; /* 0 or 1: see below                    */
} moe_shape;

/*
 * batch_invariant = 1 makes every per-token result (affinities, selection,
 * gates, expert rows, layer output) bit-identical whatever other tokens share
 * the batch and wherever the token sits in it: the property the
 * batch-invariant kernels of "DeepSeek V3 / V4 Infra" (the V4 section on
 * determinism and batch invariance) are built for. The grouped FFN and the
 * combine have it in both modes (no reduction is split across rows or
 * blocks); the router's logits GEMM splits its K reduction into slices, by
 * default as many as fill the GPU for this T, with batch_invariant = 1 into
 * a fixed count of slices of whole 128-wide chunks that d and N_r alone set
 * (eight, or four when N_r is not a multiple of 4). The bias update
 * and the load histogram are batch statistics by definition.
 */

/*
 * moe_route -- affinities, biased group-limited top-K, gates and load histogram.
 * Defined by eq. (15) (s = Sigmoid(u . e_i)), eq. (16) (selection on s + b),
 * eq. (13)-(14) (gates = selected s / their sum) of "DeepSeek_V3_Report:
 * Annotation", section "DeepSeekMoE with Auxiliary-Loss-Free Load Balancing",
 * and its section "Node-Limited Routing" (at most M groups per token).
 *   act        MOE_F32 or MOE_BF16: dtype of u and centroids.
 *   u          [T, d] token inputs.
 *   centroids  [N_r, d] expert centroid vectors e_i.
 *   bias       [N_r] fp32 expert biases b_i (selection only).
 *   topk_idx   out [T, K] int32, selected experts of each token in ascending id order.
 *   topk_gate  out [T, K] fp32, gate of each selected expert (sums to 1 per token).
 *   expert_load out [N_r] int32, number of tokens per expert (overwritten, not accumulated).
 *   scores     out [T, N_r] fp32 sigmoid affinities, or NULL (not written; with act = MOE_F32 they
 *              pass through the workspace).
 *   workspace  device scratch of at least moe_workspace_bytes(shape, ...) bytes, always
 *              required: bf16 logits are summed over K slices through it.
 * Selection compares fp32 values s + b; ties go to the lower group / expert id.
 */
moe_status moe_route(const moe_shape* shape, moe_dtype act, const void* u, const void* centroids,
                     const float* bias, int32_t* topk_idx, float* topk_gate, int32_t* expert_load,
                     float* scores, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_permute -- stable permutation of the T*K token-expert pairs to their experts
 * (the one-GPU form of the dispatch; no pair is dropped, per the section
 * "No Token-Dropping" of "DeepSeek_V3_Report: Annotation"), optionally with the
 * row gather and the online fp8 quantisation of the activations (1x128 tiles,
 * section "Fine-Grained Quantization"; scale from the current max-abs, section
 * "Online Quantization").
 *   topk_idx       [T, K] int32, as moe_route writes it (K distinct ids in [0, N_r) per token).
 *                  A pair whose id lies outside [0, N_r) or repeats an earlier id of the
 *                  same token gets no row: its row_of entry is -1 (moe_combine skips it),
 *                  expert_offsets count only the pairs that got a row, and perm_token
 *                  entries from expert_offsets[N_r] to T*K - 1 are -1.
 *   expert_offsets out [N_r + 1] int32: rows of expert e are [off[e], off[e+1]).
 *   perm_token     out [T*K] int32: token of each row (rows ordered by expert, then token).
 *   row_of         out [T*K] int32: row of pair (t, k) at index t*K + k.
 *   a              out or NULL. gather=1: [T*K, d] rows a[r] = u[perm_token[r]];
 *                  gather=0: [T, d] in token order (only with a quantised a_dtype:
 *                  the quantised u, to be gathered inside moe_grouped_ffn).
 *   a_dtype        dtype of a: act (plain copy), MOE_F8E4M3 (quantised) or
 *                  MOE_F8E4M3_POW2 (quantised with power-of-two scales: the form the
 *                  section "Low-Precision Communication" gives the activations
 *                  dispatched to the up-projection; a then feeds moe_grouped_ffn
 *                  with w = MOE_F8E4M3 like any other E4M3 operand).
 *   a_scale        out [rows of a, d/128] fp32 scales when a is quantised, else NULL.
 *                  Quantisation of a tile x: amax = max|x|; amax = 0 gives scale 1
 *                  and zero codes; else, MOE_F8E4M3: q = E4M3_rne_sat(x * fl32(448/amax)),
 *                  scale = fl32(amax/448); MOE_F8E4M3_POW2: scale = the smallest power
 *                  of two >= fl32(amax/448), q = E4M3_rne(x / scale) (x / scale is exact).
 * Deterministic: the result does not depend on the order atomics complete in.
 */
moe_status moe_permute(const moe_shape* shape, moe_dtype act, const int32_t* topk_idx, const void* u,
                       int32_t* expert_offsets, int32_t* perm_token, int32_t* row_of,
                       void* a, moe_dtype a_dtype, float* a_scale, int32_t gather,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, layouts,
 * results and errors as moe_permute. Its scratch (the per-chunk expert masks
 * and row bases) is a static 4 MiB array in the library, one per GPU, held
 * until the process ends; its device address is looked up once per device
 * on the first call made with that device current. No call allocates or
 * frees memory. Every element of the scratch a call reads is first written by
 * the same call, so nothing needs clearing between calls. Calls that overlap
 * on one GPU (on different streams or threads) share the array and race:
 * serialise them. MOE_E_UNSUPPORTED when the shape needs more scratch than
 * moe_permute_noalloc_max_scratch() bytes (ceil(T / 64) * N_r * 12 + 256;
 * e.g. T = 65536 with 256 experts needs 3 MiB).
 */
moe_status moe_permute_noalloc(const moe_shape* shape, moe_dtype act, const int32_t* topk_idx, const void* u,
                               int32_t* expert_offsets, int32_t* perm_token, int32_t* row_of, void* a,
                               moe_dtype a_dtype, float* a_scale, int32_t gather, void* stream);
size_t moe_permute_noalloc_max_scratch(void);

/*
 * moe_grouped_ffn -- per-expert SwiGLU FFN as one grouped GEMM pass over all experts:
 * y[r] = (SiLU(x W_g^T) * (x W_u^T)) W_d^T for every row r of every expert
 * (SwiGLU paragraph of "DeepSeek_V3_Report: Annotation", beta = 1; the three
 * projections cost 6*d*I FLOPs per row, "DeepSeek V3 / V4 Infra", V4 EP section).
 *   w            weight dtype: MOE_F32 (a f32), MOE_BF16 (a bf16; MOE_BF16_TILED: the same
 *                with the weights from moe_tile_weights_bf16), MOE_F8E4M3
 *                (a is fp8 with a_scale; weights fp8 with 128x128 block scales;
 *                fp32 accumulation with the scales applied per 128-wide K chunk,
 *                section "Increasing Accumulation Precision"; the SwiGLU output
 *                is re-quantised per 1x128 tile along I before the down projection)
 *                or MOE_F4E2M1 (MXFP4 expert weights, "DeepSeek V3 / V4 Infra",
 *                V4 post-training FP4 QAT; a and H as with MOE_F8E4M3, the E8M0
 *                weight scales applied by the matrix instruction, fp32 accumulation).
 *   n_experts    experts in this call (routed N_r, or N_s for the shared experts); at most 4096,
 *                2048 with bf16 or MXFP4 weights (MOE_E_UNSUPPORTED beyond).
 *   n_rows       total rows = expert_offsets[n_experts] (T*K routed, N_s*T shared).
 *   expert_offsets [n_experts + 1] int32 device array.
 *   mode, row_src  see moe_row_mode; row_src [n_rows] int32 for MOE_ROWS_GATHER, else NULL.
 *   a            input rows [a_rows, d]; a_scale [a_rows, d/128] fp32 for fp8, else NULL.
 *   w_gate_up    [n_experts, 2I, d]: gate rows [0, I) then up rows [I, 2I), K-contiguous
 *                (MOE_F8E4M3: the tiled codes of moe_quantize_weights with gate_up = 1,
 *                2I * d bytes per expert; MOE_F4E2M1: the tiled codes of
 *                moe_quantize_weights_mxfp4 with gate_up = 1, I * d bytes per expert).
 *   w_gu_scale   MOE_F8E4M3: [n_experts, 2I/128, d/128] fp32 block scales;
 *                MOE_F4E2M1: the tiled scales (gate_up = 1, 2I * d/32 bytes per expert);
 *                else NULL.
 *   w_down       [n_experts, d, I], K-contiguous (MOE_F8E4M3: tiled codes with
 *                gate_up = 0, ceil(d/256) * 256 * I bytes per expert; MOE_F4E2M1:
 *                tiled codes with gate_up = 0, ceil(d/256) * 256 * I/2 bytes per expert).
 *   w_d_scale    MOE_F8E4M3: [n_experts, d/128, I/128] fp32; MOE_F4E2M1: tiled
 *                scales (gate_up = 0, ceil(d/256) * 256 * I/32 bytes per expert); else NULL.
 *   y_dtype      MOE_F32 (only with w = MOE_F32) or MOE_BF16.
 *   y            out [n_rows, d].
 * Limits: d and I multiples of 128; with MOE_BF16, a_rows * d, n_rows * I and
 * 2 * I * d below 2^31 elements, with MOE_F8E4M3 / MOE_F4E2M1 below 2^32 and
 * d, I <= 10240 (32-bit byte offsets; MOE_F4E2M1: d, I <= 8192); otherwise
 * MOE_E_UNSUPPORTED.
 */
moe_status moe_grouped_ffn(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                           const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                           const void* a, const float* a_scale, int32_t a_rows,
                           const void* w_gate_up, const void* w_gu_scale,
                           const void* w_down, const void* w_d_scale,
                           moe_dtype y_dtype, void* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_ffn_gate_up / moe_ffn_down -- the two GEMM phases of moe_grouped_ffn as
 * separate calls, for callers that schedule or time them apart:
 * moe_grouped_ffn(...) == moe_ffn_gate_up(...) into its workspace, then moe_ffn_down(...).
 * Arguments as in moe_grouped_ffn, plus the SwiGLU output
 *   h        [n_rows, I]: fp32 (w = MOE_F32), bf16 (w = MOE_BF16) or E4M3 codes
 *            (w = MOE_F8E4M3 / MOE_F4E2M1, quantised per 1x128 tile along I with h_scale).
 *   h_scale  [n_rows, I/128] fp32 for fp8 / mxfp4, else NULL.
 *   workspace device scratch of at least 128 bytes (the counters of the
 *            kernel's dynamic work queue, cleared by the call itself); it must
 *            not overlap h or another call's workspace that is in flight.
 */
moe_status moe_ffn_gate_up(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                           const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                           const void* a, const float* a_scale, int32_t a_rows,
                           const void* w_gate_up, const void* w_gu_scale,
                           void* h, float* h_scale, void* workspace, size_t ws_bytes, void* stream);
moe_status moe_ffn_down(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                        const int32_t* expert_offsets, const void* h, const float* h_scale,
                        const void* w_down, const void* w_d_scale, moe_dtype y_dtype, void* y,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_combine -- eq. (12): out[t] = u[t] + sum_s y_shared[s*T + t] + sum_k gate[t,k] * y_routed[row_of[t*K+k]].
 * fp32 accumulation in that fixed order, one rounding to the output dtype.
 *   io        MOE_F32 or MOE_BF16: dtype of u, y_routed, y_shared and out.
 *   y_shared  [N_s*T, d], NULL iff N_s = 0.
 */
moe_status moe_combine(const moe_shape* shape, moe_dtype io, const void* u, const void* y_routed,
                       const int32_t* row_of, const float* topk_gate, const void* y_shared,
                       void* out, void* stream);

/*
 * moe_bias_update -- step-end update of the aux-loss-free bias ("DeepSeek_V3_Report:
 * Annotation", section "DeepSeekMoE with Auxiliary-Loss-Free Load Balancing"):
 * bias[i] -= gamma if expert i received more than the mean T*K/N_r pairs,
 * bias[i] += gamma if fewer, unchanged at the mean. fp32 arithmetic, in place.
 *   expert_load [N_r] int32 from moe_route.
 */
moe_status moe_bias_update(const moe_shape* shape, const int32_t* expert_load, float gamma,
                           float* bias, void* stream);

/*
 * moe_balance_stats -- complementary sequence-wise balance statistics, eq. (17)-(20) of
 * "DeepSeek_V3_Report: Annotation", section "Complementary Sequence-Wise Auxiliary Loss",
 * for each run of seq_len consecutive tokens (the last run may be shorter, T_s tokens):
 *   f_i  = N_r / (K T_s) * #{t in the run : i in topk_idx[t, :]}
 *   P_i  = (1 / T_s) * sum_t s_{i,t} / sum_j s_{j,t}
 *   loss = alpha * sum_i f_i P_i
 * The selection indicator is the routing's own choice (topk_idx, after the bias and the
 * group limit).
 *   scores    [T, N_r] fp32 affinities s (moe_route's scores output).
 *   topk_idx  [T, K] int32 from moe_route; entries outside [0, N_r) are not counted.
 *   seq_len   tokens per sequence, >= 1.
 *   f, P      out [ceil(T / seq_len), N_r] fp32; loss out [ceil(T / seq_len)] fp32.
 *   workspace at least moe_workspace_bytes(shape, ...) bytes (per-64-token partial sums).
 * fp32 arithmetic; partial sums are added in a fixed order, so results are reproducible.
 */
moe_status moe_balance_stats(const moe_shape* shape, const float* scores, const int32_t* topk_idx,
                             int32_t seq_len, float alpha, float* f, float* P, float* loss,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_quantize_weights -- 128x128 block quantisation of expert weights to E4M3
 * ("DeepSeek_V3_Report: Annotation", section "Fine-Grained Quantization") for
 * MOE_F8E4M3: for n_mats bf16 matrices [rows, cols] (multiples of 128), one fp32
 * scale per block with the same tile rule as moe_permute (scales
 * [n_mats, rows/128, cols/128]), and the codes in the tiled layout the grouped
 * FFN streams:
 *   rows go in tiles of 256, ntiles = ceil(rows / 256), tile row rw of tile t
 *   holding matrix row 256 t + rw (gate_up = 0; rows past the matrix: zero
 *   codes) or, with gate_up = 1 (rows = 2I, I a multiple of 128), j = (rw >> 5) & 3
 *   and hc = 128 t + 64 (rw >> 7) + 32 (j & 1) + (rw & 31): row hc for j < 2
 *   (gate), I + hc for j >= 2 (up);
 *   codes [n_mats][ntiles][cols/64][16384] bytes: per 64-wide K step s, the 64
 *   codes of tile row rw (K 64s .. 64s+63) at 64 rw, their 16-byte quarter c at
 *   64 rw + 16 (c ^ ((rw >> 2) & 3)).
 * Weight preparation, not part of a forward.
 */
moe_status moe_quantize_weights(int32_t n_mats, int32_t rows, int32_t cols, int32_t gate_up, const void* w_bf16,
                                void* w_codes, float* w_scale, void* stream);

/*
 * ---- Backward of the layer (bf16 weights, fp32 accumulation, fp32 weight
 * gradients). Readings of "DeepSeek_V3_Report: Annotation" (eq. (12)-(15) and
 * the FP8 framework's mixed-precision and low-precision-activation sections):
 * the selection is fixed, so the loss reaches the affinities only through the
 * gates of the selected experts and the bias gets no gradient; the gating and
 * the combine stay in high precision; the SwiGLU inputs are cached in the
 * forward (moe_ffn_gate_up_cache) and its output is recomputed in the
 * backward. One backward step: moe_combine_backward, moe_ffn_backward (routed
 * and shared experts in one call on their concatenated rows, like
 * moe_grouped_ffn), moe_route_backward, moe_input_grad.
 *
 * moe_ffn_gate_up_cache -- moe_ffn_gate_up for bf16 weights (MOE_BF16 or
 * MOE_BF16_TILED) that also writes the SwiGLU inputs gu_cache [n_rows, 2I] bf16:
 * G = a W_g^T in columns [0, I), U = a W_u^T in [I, 2I).
 */
moe_status moe_ffn_gate_up_cache(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                                 const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                                 const void* a, int32_t a_rows, const void* w_gate_up, void* h, void* gu_cache,
                                 void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_combine_backward -- from d_out [T, d] (the gradient of the layer output):
 * dy [T*K + N_s*T, d] (dy_dtype MOE_BF16, the input of both FFN backward calls, or MOE_F32),
 * dy[row_of(t,k)] = gate[t,k] * d_out[t] for the routed rows and
 * dy[T*K + s*T + t] = d_out[t] for shared expert s; d_gate [T, K] fp32,
 * d_gate[t,k] = d_out[t] . y_routed[row_of(t,k)] (fp32 sums). io (d_out, y_routed) = MOE_BF16.
 */
moe_status moe_combine_backward(const moe_shape* shape, moe_dtype io, const void* d_out, const void* y_routed,
                                const int32_t* row_of, const float* topk_gate, moe_dtype dy_dtype, void* dy,
                                float* d_gate, void* stream);

/*
 * moe_route_backward -- through the gates (eq. (13)-(14)) and the sigmoid
 * affinity (eq. (15)): per token, over its selected experts (S = sum of their
 * s), ds_k = (d_gate_k - sum_j g_j d_gate_j) / S and dz_k = ds_k s_k (1 - s_k);
 *   du_router [T, d] fp32 = sum_k dz_k e_{idx_k};
 *   d_centroids [N_r, d] fp32: row e = sum over expert e's permuted rows r (in a
 *   fixed order) of dz(r) * u[perm_token[r]] (zero for experts without rows).
 * scores, topk_idx, expert_offsets, perm_token and row_of are the forward's.
 * workspace: at least T*K*4 bytes.
 */
moe_status moe_route_backward(const moe_shape* shape, moe_dtype act, const void* u, const void* centroids,
                              const float* scores, const int32_t* topk_idx, const float* d_gate,
                              const int32_t* expert_offsets, const int32_t* perm_token, const int32_t* row_of,
                              float* du_router, float* d_centroids, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * moe_transpose_weights_bf16 -- W [n_mats][rows][cols] bf16 (rows, cols multiples
 * of 128) -> W^T [n_mats][cols][rows] in the tiled layout of moe_tile_weights_bf16
 * with gate_up = 0: the weights of the input-gradient GEMMs, which contract over
 * W's rows (W_down [E, d, I] -> [E, I, d]; W_gate_up [E, 2I, d] -> [E, d, 2I]).
 */
moe_status moe_transpose_weights_bf16(int32_t n_mats, int32_t rows, int32_t cols, const void* w_bf16,
                                      void* w_t_tiled, void* stream);

/*
 * moe_ffn_backward -- backward of the grouped SwiGLU FFN for the rows of
 * n_experts experts (expert_offsets, mode, row_src, a, a_rows as in the forward):
 *   dh = dy W_d; dG = dh U SiLU'(G), dU = dh SiLU(G) (G, U from gu_cache, SiLU' =
 *   sigma (1 + x (1 - sigma))); da [n_rows, d] bf16 = dG W_g + dU W_u;
 *   dw_down [n_experts, d, I] fp32 = dy^T h (h = SiLU(G) U recomputed);
 *   dw_gate_up [n_experts, 2I, d] fp32 = [dG | dU]^T a,
 * the weight-gradient sums running over each expert's rows (zero for experts
 * without rows). w = MOE_BF16_TILED; w_gate_up_t / w_down_t: the transposed
 * weights from moe_transpose_weights_bf16. dy [n_rows, d] bf16 (moe_combine_backward).
 * workspace: moe_ffn_backward_workspace_bytes(shape, n_rows) bytes.
 */
size_t moe_ffn_backward_workspace_bytes(const moe_shape* shape, int32_t n_rows);
moe_status moe_ffn_backward(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                            const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src, const void* a,
                            int32_t a_rows, const void* gu_cache, const void* w_gate_up_t, const void* w_down_t,
                            const void* dy, void* da, float* dw_gate_up, float* dw_down, void* workspace,
                            size_t ws_bytes, void* stream);

/*
 * moe_input_grad -- du [T, d] fp32 = d_out[t] (the residual) + du_router[t] (or 0
 * when NULL) + sum_k da[row_of(t,k)] + sum_s da[T*K + s*T + t], in that order.
 */
moe_status moe_input_grad(const moe_shape* shape, const void* d_out, const float* du_router, const void* da,
                          const int32_t* row_of, float* du, void* stream);

/*
 * ---- FP8 form of the backward (the FP8 framework of "DeepSeek_V3_Report:
 * Annotation": Fprop, Dgrad and Wgrad of every linear layer in FP8; the SwiGLU
 * inputs cached as fine-grained FP8 tiles, the SwiGLU output recomputed; the
 * Wgrad operands re-tiled from 1x128 to 128x1). Pairs with the fp8 forward
 * (MOE_F8E4M3 weights, moe_permute's E4M3 tokens).
 *
 * moe_transpose_bf16 -- W [n_mats][rows][cols] bf16 -> W^T [n_mats][cols][rows]
 * row-major (rows, cols multiples of 64). Quantising W^T with
 * moe_quantize_weights (gate_up = 0) gives the transposed 128x128 blocks with the
 * same scales: the weights of the FP8 input-gradient GEMMs.
 */
moe_status moe_transpose_bf16(int32_t n_mats, int32_t rows, int32_t cols, const void* src, void* dst, void* stream);

/*
 * moe_ffn_gate_up_cache_fp8 -- moe_ffn_gate_up for MOE_F8E4M3 that also writes the
 * SwiGLU inputs as 1x128 E4M3 tiles: gu_codes [n_rows, 2I] (G in [0, I), U in
 * [I, 2I)) and gu_scale [n_rows, 2I/128] fp32 (the forward's activation rule:
 * scale = amax / 448, code = E4M3(x * 448 / amax)). a_codes / a_scale: the 1x128
 * E4M3 tokens of moe_permute; h_codes / h_scale: the down projection's input.
 */
moe_status moe_ffn_gate_up_cache_fp8(const moe_shape* shape, int32_t n_experts, int32_t n_rows,
                                     const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                                     const void* a_codes, const float* a_scale, int32_t a_rows, const void* w_gate_up,
                                     const void* w_gu_scale, void* h_codes, float* h_scale, void* gu_codes,
                                     float* gu_scale, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_ffn_backward_fp8 -- the FP8 backward of the grouped SwiGLU FFN (rows,
 * offsets and row modes as in the forward; dy [n_rows, d] bf16 from
 * moe_combine_backward):
 *   Dgrad: dh (fp32) = Q(dy) W_d and da [n_rows, d] bf16 = Q([dG, dU]) W_gate_up on the
 *          fp8 grouped GEMM, Q = 1x128 E4M3 tiles along K, the weights as
 *          128x128 blocks of W^T (w_down_t: [n_experts][I rows, 256-row tiles][d],
 *          w_gate_up_t: [n_experts][d][2I], codes from moe_quantize_weights of
 *          moe_transpose_bf16's output, with their scales);
 *   SwiGLU backward from the cached E4M3 [G, U] (gu_codes, gu_scale), h recomputed;
 *   Wgrad: dw_down [n_experts, d, I] = R(dy)^T R(h), dw_gate_up [n_experts, 2I, d]
 *          = R([dG, dU])^T R(a) fp32, R = the 128x1 re-tiling: per column and per
 *          block of 128 consecutive rows of an expert (from its first row) one
 *          power-of-two scale, the token operand a taken from its 1x128 E4M3
 *          codes (a_codes, a_scale at the rows' source rows).
 * workspace: moe_ffn_backward_fp8_workspace_bytes(shape, n_rows, n_experts)
 * bytes. Needs 2I <= 10240.
 */
size_t moe_ffn_backward_fp8_workspace_bytes(const moe_shape* shape, int32_t n_rows, int32_t n_experts);
moe_status moe_ffn_backward_fp8(const moe_shape* shape, int32_t n_experts, int32_t n_rows,
                                const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                                const void* a_codes, const float* a_scale, int32_t a_rows, const void* gu_codes,
                                const float* gu_scale, const void* w_gate_up_t, const float* w_gate_up_t_scale,
                                const void* w_down_t, const float* w_down_t_scale, const void* dy, void* da,
                                float* dw_gate_up, float* dw_down, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_tile_weights_bf16 -- copies bf16 expert weights into the tiled layout of
 * MOE_BF16_TILED, in which every 32-wide K step of a 256-row tile is one
 * contiguous 16 KB block (the grouped FFN's load pattern). n_mats matrices
 * [rows, cols] (cols a multiple of 128) from w_bf16 to w_tiled
 * (n_mats * ceil(rows/256) * 256 * cols bf16 values, not overlapping w_bf16):
 * tile row rw of tile t holds matrix row 256 t + rw (gate_up = 0; rows past the
 * matrix are zero) or, with gate_up = 1 (rows = 2I, I a multiple of 128),
 * j = (rw >> 5) & 3 and hc = 128 t + 64 (rw >> 7) + 32 (j & 1) + (rw & 31): row
 * hc for j < 2 (gate), I + hc for j >= 2 (up). Per K step s the 64 bytes of
 * tile row rw (K 32s .. 32s+31) sit at 64 rw of the step's block, their
 * 16-byte quarter c at 64 rw + 16 (c ^ ((rw >> 2) & 3)); the blocks run
 * [n_mats][ntiles][cols/32]. Weight preparation, not part of a forward.
 */
moe_status moe_tile_weights_bf16(int32_t n_mats, int32_t rows, int32_t cols, int32_t gate_up, const void* w_bf16,
                                 void* w_tiled, void* stream);

/*
 * moe_quantize_weights_mxfp4 -- MXFP4 (OCP microscaling FP4) quantisation of
 * expert weights for MOE_F4E2M1 ("DeepSeek V3 / V4 Infra", V4 post-training FP4
 * QAT of the MoE expert weights), written in the tiled layout the grouped FFN
 * streams. For n_mats bf16 matrices [rows, cols] (cols = K, a multiple of 128),
 * per 32 consecutive values of a row: k = floor(log2(amax)) - 2 (at least -127;
 * 0 for an all-zero block), scale byte k + 127, codes E2M1 of x * 2^-k, round
 * to nearest with ties to the even code, saturating at 6, sign bit from x.
 *
 * Layout. Rows go in tiles of 256, ntiles = ceil(rows / 256); tile row rw
 * (0..255) of tile t holds matrix row
 *   gate_up = 0:  256 t + rw (rows past the matrix: codes 0, scale byte 127);
 *   gate_up = 1 (rows = 2I, I a multiple of 128, the gate rows then the up
 *   rows): with j = (rw >> 5) & 3 and hc = 128 t + 64 (rw >> 7) + 32 (j & 1) +
 *   (rw & 31), row hc for j < 2 (gate) and I + hc for j >= 2 (up), so that a
 *   tile holds the gate and up rows of 128 H columns.
 * codes  [n_mats][ntiles][K/64][8192] bytes: per 64-wide K step, the 32 code
 *        bytes of K values 64s .. 64s+63 of tile row rw start at 32 rw; their
 *        16-byte halves k16 = 0, 1 (K 64s + 32 k16 .. +31) sit at byte
 *        32 rw + 16 (k16 ^ ((rw >> 3) & 1)); two codes per byte, the even K
 *        index in the low nibble.
 * scales [n_mats][ntiles][K/128][4][256] bytes: scale of tile row rw for the
 *        32-value block 4c + b at [c][b][rw].
 * Weight preparation, not part of a forward.
 */
moe_status moe_quantize_weights_mxfp4(int32_t n_mats, int32_t rows, int32_t cols, int32_t gate_up,
                                      const void* w_bf16, void* w_codes, void* w_scale, void* stream);

/* Host: bytes of workspace that any single call above needs for this shape,
 * with moe_grouped_ffn sized for T*(K + N_s) rows: the routed and the shared
 * experts in one call (shared expert s as one more expert whose rows are all
 * T tokens). One workspace can serve all calls issued in order on one stream. */
size_t moe_workspace_bytes(const moe_shape* shape, moe_dtype gemm);

/* Host: message of the calling thread's last non-OK status ("" if none). */
const char* moe_last_error(void);

/* Host: library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
