// The C ABI of include/moe.h: argument validation on the host (before any
// HIP call), workspace sizing, dispatch to the launchers, error reporting.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <string>

#include "launch.h"
#include "sched.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

bool sync_debug() {
  static const bool on = [] {
    const char* v = std::getenv("MOE_SYNC_DEBUG");
    return v && v[0] == '1';
  }();
  return on;
}

moe_status finish(hipError_t e, const char* what, hipStream_t st) {
  if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

#define REQUIRE(cond, ...)                          \
  do {                                              \
    if (!(cond)) return fail(MOE_E_INVALID, __VA_ARGS__); \
  } while (0)
#define SUPPORT(cond, ...)                              \
  do {                                                  \
    if (!(cond)) return fail(MOE_E_UNSUPPORTED, __VA_ARGS__); \
  } while (0)

moe_status check_shape(const moe_shape* s) {
  REQUIRE(s != nullptr, "shape is NULL");
  REQUIRE(s->T > 0 && s->d > 0 && s->n_routed > 0 && s->n_groups > 0 && s->topk_groups > 0 &&
              s->group_topn > 0 && s->topk > 0 && s->inter > 0 && s->n_shared >= 0,
          "non-positive size in shape (T=%d d=%d N_r=%d G=%d M=%d topn=%d K=%d N_s=%d I=%d)", s->T, s->d,
          s->n_routed, s->n_groups, s->topk_groups, s->group_topn, s->topk, s->n_shared, s->inter);
  REQUIRE(s->batch_invariant == 0 || s->batch_invariant == 1, "batch_invariant must be 0 or 1 (got %d)",
          s->batch_invariant);
  REQUIRE(s->n_routed % s->n_groups == 0, "n_routed (%d) is not a multiple of n_groups (%d)", s->n_routed,
          s->n_groups);
  REQUIRE(s->topk_groups <= s->n_groups, "topk_groups (%d) > n_groups (%d)", s->topk_groups, s->n_groups);
  const int S = s->n_routed / s->n_groups;
  REQUIRE(s->group_topn <= S, "group_topn (%d) > group size (%d)", s->group_topn, S);
  REQUIRE(s->topk <= s->topk_groups * S, "topk (%d) > topk_groups * group size (%d)", s->topk,
          s->topk_groups * S);
  SUPPORT(s->d % 128 == 0, "d (%d) must be a multiple of 128", s->d);
  SUPPORT(s->inter % 128 == 0, "inter (%d) must be a multiple of 128", s->inter);
  SUPPORT(s->topk <= 16, "topk (%d) > 16", s->topk);
  SUPPORT(s->n_routed <= 1024, "n_routed (%d) > 1024", s->n_routed);
  SUPPORT(s->n_groups <= 64, "n_groups (%d) > 64", s->n_groups);
  SUPPORT(s->group_topn <= 4, "group_topn (%d) > 4", s->group_topn);
  SUPPORT(static_cast<long long>(s->T) * s->topk < (1LL << 31) && static_cast<long long>(s->T) * s->n_shared < (1LL << 31),
          "T*K or T*N_s does not fit int32");
  return MOE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

std::mutex g_cu_mutex;
int g_cu[64];

// Scratch of moe_permute_noalloc: one copy per GPU, held until the process
// ends. Host code never uses the array's name as an address (on the host it is
// a stand-in symbol): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept per device.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[64];

moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_E_HIP, "permute_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_E_UNSUPPORTED, "permute_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_E_HIP, "permute_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

namespace moe {

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(g_cu_mutex);
  if (g_cu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu[dev] = n;
  }
  return g_cu[dev];
}

__global__ void queue_reset_kernel(int* q) {
  if (threadIdx.x < kQueueInts) q[threadIdx.x] = 0;
}

hipError_t launch_queue_reset(int* q, hipStream_t st) {
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, st, q);
  return hipGetLastError();
}

size_t ffn_queue_offset(moe_dtype w, int n_rows, int I) {
  const size_t n = static_cast<size_t>(n_rows) * I;
  if (w == MOE_F32) return align256(n * 4);
  if (w == MOE_BF16 || w == MOE_BF16_TILED) return align256(n * 2);
  return align256(n) + align256(static_cast<size_t>(n_rows) * (I / 128) * 4);
}

size_t ffn_ws_bytes(moe_dtype w, int n_rows, int I) { return ffn_queue_offset(w, n_rows, I) + 2 * kFfnQueueBytes; }

}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe-gfx950 0.1"; }

size_t moe_workspace_bytes(const moe_shape* shape, moe_dtype gemm) {
  if (!shape || check_shape(shape) != MOE_OK) return 0;
  const moe::Shape s = moe::to_shape(*shape);
  const size_t route = align256(moe::route_ws_bytes(s, MOE_BF16));
  const size_t bal = align256(moe::balance_ws_bytes(s, 1));     // seq_len = 1 needs the most
  const size_t perm = align256(moe::permute_ws_bytes(s));
  const int rows = s.T * (s.K + s.Ns);   // routed and shared experts in one grouped call
  const size_t ffn = moe::ffn_ws_bytes(gemm, rows, s.I);
  size_t m = route > perm ? route : perm;
  m = m > bal ? m : bal;
  return m > ffn ? m : ffn;
}

moe_status moe_route(const moe_shape* shape, moe_dtype act, const void* u, const void* centroids,
                     const float* bias, int32_t* topk_idx, float* topk_gate, int32_t* expert_load, float* scores,
                     void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(act == MOE_F32 || act == MOE_BF16, "route: act must be MOE_F32 or MOE_BF16 (got %d)", static_cast<int>(act));
  REQUIRE(u && centroids && bias && topk_idx && topk_gate && expert_load, "route: a required pointer is NULL");
  const moe::Shape s = moe::to_shape(*shape);
  const size_t need = moe::route_ws_bytes(s, act);
  if (!workspace || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "route: workspace of %zu bytes < %zu needed", ws_bytes, need);
  // the fp32 path computes the affinities in one kernel and selects in the next, so they go through memory:
  // the workspace when the caller does not want them; the bf16 path writes them only when asked
  if (!scores && act != MOE_BF16) scores = static_cast<float*>(workspace);
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_route(s, act, u, centroids, bias, topk_idx, topk_gate, expert_load, scores, workspace, st),
                "moe_route", st);
}

moe_status moe_permute(const moe_shape* shape, moe_dtype act, const int32_t* topk_idx, const void* u,
                       int32_t* expert_offsets, int32_t* perm_token, int32_t* row_of, void* a, moe_dtype a_dtype,
                       float* a_scale, int32_t gather, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(topk_idx && expert_offsets && perm_token && row_of, "permute: a required pointer is NULL");
  const moe::Shape s = moe::to_shape(*shape);
  if (a) {
    REQUIRE(u != nullptr, "permute: u is NULL but an output a is requested");
    REQUIRE(act == MOE_F32 || act == MOE_BF16, "permute: act must be MOE_F32 or MOE_BF16");
    const bool quant = a_dtype == MOE_F8E4M3 || a_dtype == MOE_F8E4M3_POW2;
    REQUIRE(a_dtype == act || quant, "permute: a_dtype must equal act or be MOE_F8E4M3 / MOE_F8E4M3_POW2");
    REQUIRE(!quant || a_scale != nullptr, "permute: fp8 output needs a_scale");
    REQUIRE(gather == 0 || gather == 1, "permute: gather must be 0 or 1");
    REQUIRE(gather == 1 || quant, "permute: gather=0 is only meaningful for fp8 quantisation");
  }
  const size_t need = moe::permute_ws_bytes(s);
  if (!workspace || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "permute: workspace of %zu bytes < %zu needed", ws_bytes, need);
  auto st = static_cast<hipStream_t>(stream);
  hipError_t e = moe::launch_permute_maps(s, topk_idx, expert_offsets, perm_token, row_of, workspace, st);
  if (e == hipSuccess && a) {
    const int rows = gather ? s.T * s.K : s.T;
    e = moe::launch_rows_copy(rows, s.d, act, u, s.T, gather ? perm_token : nullptr, a_dtype, a, a_scale, st);
  }
  return finish(e, "moe_permute", st);
}

moe_status moe_permute_noalloc(const moe_shape* shape, moe_dtype act, const int32_t* topk_idx, const void* u,
                               int32_t* expert_offsets, int32_t* perm_token, int32_t* row_of, void* a,
                               moe_dtype a_dtype, float* a_scale, int32_t gather, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  const size_t need = moe::permute_ws_bytes(moe::to_shape(*shape));
  if (need > kScratchBytes)
    return fail(MOE_E_UNSUPPORTED,
                "permute_noalloc: T=%d with %d experts needs %zu bytes of scratch, above its static %zu; "
                "call moe_permute with a workspace",
                shape->T, shape->n_routed, need, kScratchBytes);
  void* ws = nullptr;
  if (moe_status st = scratch_address(&ws); st != MOE_OK) return st;
  return moe_permute(shape, act, topk_idx, u, expert_offsets, perm_token, row_of, a, a_dtype, a_scale, gather, ws,
                     kScratchBytes, stream);
}

size_t moe_permute_noalloc_max_scratch(void) { return kScratchBytes; }

}  // extern "C"

namespace {

// Validation shared by the grouped FFN calls (phase: 0 both, 1 gate/up, 2 down).
moe_status check_ffn(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                     const int32_t* offsets, int phase) {
  REQUIRE(shape != nullptr, "shape is NULL");
  const int d = shape->d, I = shape->inter;
  REQUIRE(d > 0 && I > 0, "grouped_ffn: d and inter must be positive");
  SUPPORT(d % 128 == 0 && I % 128 == 0, "grouped_ffn: d (%d) and inter (%d) must be multiples of 128", d, I);
  REQUIRE(n_experts > 0 && n_rows > 0, "grouped_ffn: n_experts and n_rows must be positive");
  SUPPORT(n_experts <= 4096, "grouped_ffn: n_experts (%d) > 4096", n_experts);
  // the bf16 and mxfp4 kernels keep their per-expert schedule table in LDS beside a larger ring
  SUPPORT((w != MOE_BF16 && w != MOE_BF16_TILED && w != MOE_F4E2M1) || n_experts <= 2048,
          "grouped_ffn: the bf16 and mxfp4 paths take at most 2048 experts per call (n_experts = %d)", n_experts);
  SUPPORT(static_cast<long long>(n_rows) * (d > I ? d : I) < (1LL << 40), "grouped_ffn: too many rows");
  REQUIRE(offsets != nullptr, "grouped_ffn: expert_offsets is NULL");
  REQUIRE(w == MOE_F32 || w == MOE_BF16 || w == MOE_BF16_TILED || w == MOE_F8E4M3 || w == MOE_F4E2M1,
          "grouped_ffn: bad weight dtype %d", static_cast<int>(w));
  const bool q8 = w == MOE_F8E4M3 || w == MOE_F4E2M1;   // E4M3 activations and H
  SUPPORT(!q8 || (d <= 10240 && I <= 10240), "grouped_ffn: the fp8 / mxfp4 paths need d and inter <= 10240");
  SUPPORT(w != MOE_F4E2M1 || (d <= 8192 && I <= 8192), "grouped_ffn: the mxfp4 path needs d and inter <= 8192");
  // the fp8 / mxfp4 kernels address codes and scales through 32-bit byte offsets
  SUPPORT(!q8 || (static_cast<long long>(n_rows) * I < (1LL << 32) && static_cast<long long>(2 * I) * d < (1LL << 32)),
          "grouped_ffn: fp8 / mxfp4 paths need n_rows * inter and 2 * inter * d below 2^32");
  // the bf16 kernels address H and one expert's weight matrices through 32-bit byte offsets
  SUPPORT((w != MOE_BF16 && w != MOE_BF16_TILED) || (static_cast<long long>(n_rows) * I * 2 < (1LL << 32) &&
                                                     static_cast<long long>(2 * I) * d * 2 < (1LL << 32)),
          "grouped_ffn: bf16 path needs n_rows * inter and 2 * inter * d below 2^31 elements");
  (void)phase;
  return MOE_OK;
}

moe_status check_gate_up(const moe_shape* shape, moe_dtype w, moe_row_mode mode, const int32_t* row_src,
                         const void* a, const float* a_scale, int32_t a_rows, const void* w_gate_up,
                         const void* w_gu_scale) {
  REQUIRE(a && w_gate_up, "grouped_ffn: a or w_gate_up is NULL");
  REQUIRE(a_rows > 0, "grouped_ffn: a_rows must be positive");
  SUPPORT((w != MOE_BF16 && w != MOE_BF16_TILED) || static_cast<long long>(a_rows) * shape->d * 2 < (1LL << 32),
          "grouped_ffn: bf16 path needs a_rows * d below 2^31 elements");
  SUPPORT((w != MOE_F8E4M3 && w != MOE_F4E2M1) || static_cast<long long>(a_rows) * shape->d < (1LL << 32),
          "grouped_ffn: fp8 / mxfp4 paths need a_rows * d below 2^32");
  REQUIRE(mode == MOE_ROWS_DIRECT || mode == MOE_ROWS_GATHER || mode == MOE_ROWS_SEGMENT,
          "grouped_ffn: bad row mode %d", static_cast<int>(mode));
  REQUIRE(mode != MOE_ROWS_GATHER || row_src != nullptr, "grouped_ffn: MOE_ROWS_GATHER needs row_src");
  if (w == MOE_F8E4M3 || w == MOE_F4E2M1)
    REQUIRE(a_scale && w_gu_scale, "grouped_ffn: fp8 / mxfp4 need a_scale and w_gu_scale");
  return MOE_OK;
}

moe_status check_down(moe_dtype w, const void* w_down, const void* w_d_scale, moe_dtype y_dtype, const void* y) {
  REQUIRE(w_down && y, "grouped_ffn: w_down or y is NULL");
  REQUIRE(y_dtype == MOE_BF16 || (y_dtype == MOE_F32 && w == MOE_F32),
          "grouped_ffn: y_dtype must be MOE_BF16 (or MOE_F32 with MOE_F32 weights)");
  if (w == MOE_F8E4M3 || w == MOE_F4E2M1) REQUIRE(w_d_scale != nullptr, "grouped_ffn: fp8 / mxfp4 need w_d_scale");
  return MOE_OK;
}

hipError_t run_gate_up(moe_dtype w, const moe::FfnArgs& p, hipStream_t st) {
  if (w == MOE_F32) return moe::launch_ffn_f32_gate_up(p, st);
  if (w == MOE_BF16 || w == MOE_BF16_TILED) return moe::launch_ffn_bf16_gate_up(p, st, w == MOE_BF16_TILED);
  if (w == MOE_F4E2M1) return moe::launch_ffn_fp4_gate_up(p, st);
  return moe::launch_ffn_fp8_gate_up(p, st);
}

hipError_t run_down(moe_dtype w, const moe::FfnArgs& p, hipStream_t st) {
  if (w == MOE_F32) return moe::launch_ffn_f32_down(p, st);
  if (w == MOE_BF16 || w == MOE_BF16_TILED) return moe::launch_ffn_bf16_down(p, st, w == MOE_BF16_TILED);
  if (w == MOE_F4E2M1) return moe::launch_ffn_fp4_down(p, st);
  return moe::launch_ffn_fp8_down(p, st);
}

}  // namespace

extern "C" {

moe_status moe_grouped_ffn(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                           const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src, const void* a,
                           const float* a_scale, int32_t a_rows, const void* w_gate_up, const void* w_gu_scale,
                           const void* w_down, const void* w_d_scale, moe_dtype y_dtype, void* y, void* workspace,
                           size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, w, n_experts, n_rows, expert_offsets, 0); r != MOE_OK) return r;
  if (moe_status r = check_gate_up(shape, w, mode, row_src, a, a_scale, a_rows, w_gate_up, w_gu_scale); r != MOE_OK)
    return r;
  if (moe_status r = check_down(w, w_down, w_d_scale, y_dtype, y); r != MOE_OK) return r;
  const int d = shape->d, I = shape->inter;
  const size_t need = moe::ffn_ws_bytes(w, n_rows, I);
  if (!workspace || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "grouped_ffn: workspace of %zu bytes < %zu needed", ws_bytes, need);
  float* h_scale = nullptr;
  if (w == MOE_F8E4M3 || w == MOE_F4E2M1)
    h_scale = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(static_cast<size_t>(n_rows) * I));
  int* queue = reinterpret_cast<int*>(static_cast<char*>(workspace) + moe::ffn_queue_offset(w, n_rows, I));
  moe::FfnArgs p{d, I, n_experts, n_rows, a_rows, expert_offsets, mode, row_src, a, a_scale, w_gate_up, w_gu_scale,
                 w_down, w_d_scale, y_dtype, y, workspace, h_scale, queue};
  auto st = static_cast<hipStream_t>(stream);
  hipError_t e = run_gate_up(w, p, st);
  p.queue = queue + moe::kFfnQueueBytes / sizeof(int);
  if (e == hipSuccess) e = run_down(w, p, st);
  return finish(e, "moe_grouped_ffn", st);
}

moe_status moe_ffn_gate_up(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                           const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src, const void* a,
                           const float* a_scale, int32_t a_rows, const void* w_gate_up, const void* w_gu_scale,
                           void* h, float* h_scale, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, w, n_experts, n_rows, expert_offsets, 1); r != MOE_OK) return r;
  if (moe_status r = check_gate_up(shape, w, mode, row_src, a, a_scale, a_rows, w_gate_up, w_gu_scale); r != MOE_OK)
    return r;
  REQUIRE(h != nullptr, "ffn_gate_up: h is NULL");
  REQUIRE((w != MOE_F8E4M3 && w != MOE_F4E2M1) || h_scale != nullptr, "ffn_gate_up: fp8 / mxfp4 need h_scale");
  if (!workspace || ws_bytes < moe::kFfnQueueBytes)
    return fail(MOE_E_WORKSPACE, "ffn_gate_up: workspace of %zu bytes < %zu needed", ws_bytes, moe::kFfnQueueBytes);
  moe::FfnArgs p{shape->d, shape->inter, n_experts, n_rows, a_rows, expert_offsets, mode, row_src, a, a_scale,
                 w_gate_up, w_gu_scale, nullptr, nullptr, MOE_BF16, nullptr, h, h_scale, static_cast<int*>(workspace)};
  auto st = static_cast<hipStream_t>(stream);
  return finish(run_gate_up(w, p, st), "moe_ffn_gate_up", st);
}

moe_status moe_ffn_down(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                        const int32_t* expert_offsets, const void* h, const float* h_scale, const void* w_down,
                        const void* w_d_scale, moe_dtype y_dtype, void* y, void* workspace, size_t ws_bytes,
                        void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, w, n_experts, n_rows, expert_offsets, 2); r != MOE_OK) return r;
  if (moe_status r = check_down(w, w_down, w_d_scale, y_dtype, y); r != MOE_OK) return r;
  REQUIRE(h != nullptr, "ffn_down: h is NULL");
  REQUIRE((w != MOE_F8E4M3 && w != MOE_F4E2M1) || h_scale != nullptr, "ffn_down: fp8 / mxfp4 need h_scale");
  if (!workspace || ws_bytes < moe::kFfnQueueBytes)
    return fail(MOE_E_WORKSPACE, "ffn_down: workspace of %zu bytes < %zu needed", ws_bytes, moe::kFfnQueueBytes);
  moe::FfnArgs p{shape->d, shape->inter, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr,
                 nullptr, nullptr, nullptr, nullptr, w_down, w_d_scale, y_dtype, y, const_cast<void*>(h),
                 const_cast<float*>(h_scale), static_cast<int*>(workspace)};
  auto st = static_cast<hipStream_t>(stream);
  return finish(run_down(w, p, st), "moe_ffn_down", st);
}

moe_status moe_balance_stats(const moe_shape* shape, const float* scores, const int32_t* topk_idx, int32_t seq_len,
                             float alpha, float* f, float* P, float* loss, void* workspace, size_t ws_bytes,
                             void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(scores && topk_idx && f && P && loss, "balance_stats: a required pointer is NULL");
  REQUIRE(seq_len >= 1, "balance_stats: seq_len (%d) must be positive", seq_len);
  const moe::Shape s = moe::to_shape(*shape);
  const size_t need = moe::balance_ws_bytes(s, seq_len);
  if (!workspace || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "balance_stats: workspace of %zu bytes < %zu needed", ws_bytes, need);
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_balance_stats(s, scores, topk_idx, seq_len, alpha, f, P, loss, workspace, st),
                "moe_balance_stats", st);
}

moe_status moe_combine(const moe_shape* shape, moe_dtype io, const void* u, const void* y_routed,
                       const int32_t* row_of, const float* topk_gate, const void* y_shared, void* out, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(io == MOE_F32 || io == MOE_BF16, "combine: io must be MOE_F32 or MOE_BF16");
  REQUIRE(u && y_routed && row_of && topk_gate && out, "combine: a required pointer is NULL");
  REQUIRE(shape->n_shared == 0 || y_shared != nullptr, "combine: y_shared is NULL with n_shared = %d",
          shape->n_shared);
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_combine(moe::to_shape(*shape), io, u, y_routed, row_of, topk_gate,
                                    shape->n_shared ? y_shared : nullptr, out, st),
                "moe_combine", st);
}

moe_status moe_bias_update(const moe_shape* shape, const int32_t* expert_load, float gamma, float* bias,
                           void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(expert_load && bias, "bias_update: a required pointer is NULL");
  REQUIRE(gamma == gamma && gamma >= 0.0f, "bias_update: gamma must be a non-negative number");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_bias_update(moe::to_shape(*shape), expert_load, gamma, bias, st), "moe_bias_update",
                st);
}

moe_status moe_quantize_weights(int32_t n_mats, int32_t rows, int32_t cols, int32_t gate_up, const void* w_bf16,
                                void* w_codes, float* w_scale, void* stream) {
  g_err.clear();
  REQUIRE(n_mats > 0 && rows > 0 && cols > 0, "quantize_weights: sizes must be positive");
  REQUIRE(gate_up == 0 || gate_up == 1, "quantize_weights: gate_up must be 0 or 1");
  SUPPORT(rows % 128 == 0 && cols % 128 == 0, "quantize_weights: rows (%d) and cols (%d) must be multiples of 128",
          rows, cols);
  SUPPORT(!gate_up || rows % 256 == 0, "quantize_weights: gate_up needs rows = 2I with I a multiple of 128");
  REQUIRE(w_bf16 && w_codes && w_scale, "quantize_weights: a required pointer is NULL");
  SUPPORT(static_cast<long long>(n_mats) * (rows / 128) * (cols / 128) < (1LL << 31), "quantize_weights: too many blocks");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_quantize_weights(n_mats, rows, cols, gate_up, w_bf16, w_codes, w_scale, st),
                "moe_quantize_weights", st);
}

moe_status moe_tile_weights_bf16(int32_t n_mats, int32_t rows, int32_t cols, int32_t gate_up, const void* w_bf16,
                                 void* w_tiled, void* stream) {
  g_err.clear();
  REQUIRE(n_mats > 0 && rows > 0 && cols > 0, "tile_weights_bf16: sizes must be positive");
  REQUIRE(gate_up == 0 || gate_up == 1, "tile_weights_bf16: gate_up must be 0 or 1");
  SUPPORT(cols % 128 == 0, "tile_weights_bf16: cols (%d) must be a multiple of 128", cols);
  SUPPORT(!gate_up || rows % 256 == 0, "tile_weights_bf16: gate_up needs rows = 2I with I a multiple of 128");
  REQUIRE(w_bf16 && w_tiled, "tile_weights_bf16: a required pointer is NULL");
  REQUIRE(w_bf16 != w_tiled, "tile_weights_bf16: the copy cannot be made in place");
  SUPPORT(static_cast<long long>(n_mats) * (rows + 255) * cols < (1LL << 40), "tile_weights_bf16: too many values");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_tile_weights_bf16(n_mats, rows, cols, gate_up, w_bf16, w_tiled, st),
                "moe_tile_weights_bf16", st);
}

moe_status moe_quantize_weights_mxfp4(int32_t n_mats, int32_t rows, int32_t cols, int32_t gate_up, const void* w_bf16,
                                      void* w_codes, void* w_scale, void* stream) {
  g_err.clear();
  REQUIRE(n_mats > 0 && rows > 0 && cols > 0, "quantize_weights_mxfp4: sizes must be positive");
  REQUIRE(gate_up == 0 || gate_up == 1, "quantize_weights_mxfp4: gate_up must be 0 or 1");
  SUPPORT(cols % 128 == 0, "quantize_weights_mxfp4: cols (%d) must be a multiple of 128", cols);
  SUPPORT(!gate_up || rows % 256 == 0, "quantize_weights_mxfp4: gate_up needs rows = 2I with I a multiple of 128");
  REQUIRE(w_bf16 && w_codes && w_scale, "quantize_weights_mxfp4: a required pointer is NULL");
  SUPPORT(static_cast<long long>(n_mats) * (rows + 255) * cols < (1LL << 40), "quantize_weights_mxfp4: too many values");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_quantize_weights_mxfp4(n_mats, rows, cols, gate_up, w_bf16, w_codes, w_scale, st),
                "moe_quantize_weights_mxfp4", st);
}

// ---------------------------------------------------------------- backward

moe_status moe_ffn_gate_up_cache(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                                 const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                                 const void* a, int32_t a_rows, const void* w_gate_up, void* h, void* gu_cache,
                                 void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, w, n_experts, n_rows, expert_offsets, 1); r != MOE_OK) return r;
  REQUIRE(w == MOE_BF16 || w == MOE_BF16_TILED, "ffn_gate_up_cache: the SwiGLU-input cache needs bf16 weights");
  if (moe_status r = check_gate_up(shape, w, mode, row_src, a, nullptr, a_rows, w_gate_up, nullptr); r != MOE_OK)
    return r;
  REQUIRE(h != nullptr && gu_cache != nullptr, "ffn_gate_up_cache: h or gu_cache is NULL");
  if (!workspace || ws_bytes < moe::kFfnQueueBytes)
    return fail(MOE_E_WORKSPACE, "ffn_gate_up_cache: workspace of %zu bytes < %zu needed", ws_bytes,
                moe::kFfnQueueBytes);
  moe::FfnArgs p{shape->d, shape->inter, n_experts, n_rows, a_rows, expert_offsets, mode, row_src, a, nullptr,
                 w_gate_up, nullptr, nullptr, nullptr, MOE_BF16, nullptr, h, nullptr, static_cast<int*>(workspace)};
  p.gu_cache = gu_cache;
  auto st = static_cast<hipStream_t>(stream);
  return finish(run_gate_up(w, p, st), "moe_ffn_gate_up_cache", st);
}

moe_status moe_combine_backward(const moe_shape* shape, moe_dtype io, const void* d_out, const void* y_routed,
                                const int32_t* row_of, const float* topk_gate, moe_dtype dy_dtype, void* dy,
                                float* d_gate, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(io == MOE_BF16, "combine_backward: io must be MOE_BF16");
  REQUIRE(dy_dtype == MOE_BF16 || dy_dtype == MOE_F32, "combine_backward: dy_dtype must be MOE_BF16 or MOE_F32");
  REQUIRE(d_out && y_routed && row_of && topk_gate && dy && d_gate, "combine_backward: a required pointer is NULL");
  SUPPORT(shape->d % 2 == 0, "combine_backward: d must be even");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_combine_backward(moe::to_shape(*shape), d_out, y_routed, row_of, topk_gate, dy,
                                             dy_dtype == MOE_F32, d_gate, st),
                "moe_combine_backward", st);
}

moe_status moe_route_backward(const moe_shape* shape, moe_dtype act, const void* u, const void* centroids,
                              const float* scores, const int32_t* topk_idx, const float* d_gate,
                              const int32_t* expert_offsets, const int32_t* perm_token, const int32_t* row_of,
                              float* du_router, float* d_centroids, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(act == MOE_F32 || act == MOE_BF16, "route_backward: act must be MOE_F32 or MOE_BF16");
  REQUIRE(u && centroids && scores && topk_idx && d_gate && expert_offsets && perm_token && row_of && du_router &&
              d_centroids,
          "route_backward: a required pointer is NULL");
  const size_t need = static_cast<size_t>(shape->T) * shape->topk * sizeof(float);
  if (!workspace || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "route_backward: workspace of %zu bytes < %zu needed", ws_bytes, need);
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_route_backward(moe::to_shape(*shape), act, u, centroids, scores, topk_idx, d_gate,
                                           expert_offsets, perm_token, row_of, du_router, d_centroids,
                                           static_cast<float*>(workspace), st),
                "moe_route_backward", st);
}

moe_status moe_transpose_weights_bf16(int32_t n_mats, int32_t rows, int32_t cols, const void* w_bf16, void* w_t_tiled,
                                      void* stream) {
  g_err.clear();
  REQUIRE(n_mats > 0 && rows > 0 && cols > 0, "transpose_weights_bf16: sizes must be positive");
  SUPPORT(rows % 128 == 0 && cols % 128 == 0, "transpose_weights_bf16: rows (%d) and cols (%d) must be multiples of 128",
          rows, cols);
  REQUIRE(w_bf16 && w_t_tiled && w_bf16 != w_t_tiled, "transpose_weights_bf16: bad pointers");
  SUPPORT(static_cast<long long>(n_mats) * (rows / 32) * ((cols + 255) / 256) < (1LL << 31),
          "transpose_weights_bf16: too many blocks");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_transpose_tile_bf16(n_mats, rows, cols, w_bf16, w_t_tiled, st), "moe_transpose_weights_bf16",
                st);
}

size_t moe_ffn_backward_workspace_bytes(const moe_shape* shape, int32_t n_rows) {
  if (!shape || n_rows < 0 || shape->inter <= 0) return 0;
  const size_t r = static_cast<size_t>(n_rows), I = static_cast<size_t>(shape->inter);
  return align256(r * I * 2) + align256(r * 2 * I * 2) + align256(r * I * 2) + 2 * moe::kFfnQueueBytes;
}

moe_status moe_ffn_backward(const moe_shape* shape, moe_dtype w, int32_t n_experts, int32_t n_rows,
                            const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src, const void* a,
                            int32_t a_rows, const void* gu_cache, const void* w_gate_up_t, const void* w_down_t,
                            const void* dy, void* da, float* dw_gate_up, float* dw_down, void* workspace,
                            size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, w, n_experts, n_rows, expert_offsets, 0); r != MOE_OK) return r;
  REQUIRE(w == MOE_BF16_TILED, "ffn_backward: w must be MOE_BF16_TILED (weights from moe_transpose_weights_bf16)");
  REQUIRE(a && gu_cache && w_gate_up_t && w_down_t && dy && da && dw_gate_up && dw_down,
          "ffn_backward: a required pointer is NULL");
  REQUIRE(a_rows > 0, "ffn_backward: a_rows must be positive");
  REQUIRE(mode == MOE_ROWS_DIRECT || mode == MOE_ROWS_GATHER || mode == MOE_ROWS_SEGMENT,
          "ffn_backward: bad row mode %d", static_cast<int>(mode));
  REQUIRE(mode != MOE_ROWS_GATHER || row_src != nullptr, "ffn_backward: MOE_ROWS_GATHER needs row_src");
  const int d = shape->d, I = shape->inter;
  SUPPORT(static_cast<long long>(n_rows) * 2 * I * 2 < (1LL << 32) && static_cast<long long>(n_rows) * d * 2 < (1LL << 32),
          "ffn_backward: n_rows * 2I and n_rows * d must stay below 2^31 elements");
  SUPPORT(mode != MOE_ROWS_GATHER || static_cast<long long>(a_rows) * d * 2 < (1LL << 32) - 256,
          "ffn_backward: a gathered a must stay below 4 GiB");
  const size_t need = moe_ffn_backward_workspace_bytes(shape, n_rows);
  if (!workspace || ws_bytes < need)
    return fail(MOE_E_WORKSPACE, "ffn_backward: workspace of %zu bytes < %zu needed", ws_bytes, need);
  char* ws = static_cast<char*>(workspace);
  const size_t r = static_cast<size_t>(n_rows);
  void* dh = ws;
  void* dgu = ws + align256(r * I * 2);
  void* h = ws + align256(r * I * 2) + align256(r * 2 * I * 2);
  int* q = reinterpret_cast<int*>(ws + align256(r * I * 2) + align256(r * 2 * I * 2) + align256(r * I * 2));
  auto st = static_cast<hipStream_t>(stream);
  // dh = dy . W_d: the down-projection kernel with W_d^T (I output rows, K = d)
  moe::FfnArgs p1{I, d, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, nullptr, nullptr,
                  nullptr, nullptr, w_down_t, nullptr, MOE_BF16, dh, const_cast<void*>(dy), nullptr, q};
  hipError_t e = moe::launch_ffn_bf16_down(p1, st, true);
  if (e == hipSuccess) e = moe::launch_swiglu_backward(n_rows, I, dh, gu_cache, dgu, h, st);
  // da = [dG | dU] . W_gate_up: the same kernel with W_gate_up^T (d output rows, K = 2I)
  moe::FfnArgs p2{d, 2 * I, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, nullptr, nullptr,
                  nullptr, nullptr, w_gate_up_t, nullptr, MOE_BF16, da, dgu, nullptr, q + moe::kQueueInts};
  if (e == hipSuccess) e = moe::launch_ffn_bf16_down(p2, st, true);
  // weight gradients: dW_d = dy^T h, dW_gate_up = [dG | dU]^T a
  if (e == hipSuccess)
    e = moe::launch_wgrad(d, I, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, dy, h, dw_down,
                          st);
  if (e == hipSuccess)
    e = moe::launch_wgrad(2 * I, d, n_experts, n_rows, a_rows, expert_offsets, mode, row_src, dgu, a, dw_gate_up, st);
  return finish(e, "moe_ffn_backward", st);
}

moe_status moe_input_grad(const moe_shape* shape, const void* d_out, const float* du_router, const void* da,
                          const int32_t* row_of, float* du, void* stream) {
  g_err.clear();
  if (moe_status st = check_shape(shape); st != MOE_OK) return st;
  REQUIRE(d_out && da && row_of && du, "input_grad: a required pointer is NULL");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_input_grad(moe::to_shape(*shape), d_out, du_router, da, row_of, du, st), "moe_input_grad",
                st);
}


moe_status moe_transpose_bf16(int32_t n_mats, int32_t rows, int32_t cols, const void* src, void* dst, void* stream) {
  g_err.clear();
  REQUIRE(n_mats > 0 && rows > 0 && cols > 0, "transpose_bf16: sizes must be positive");
  SUPPORT(rows % 64 == 0 && cols % 64 == 0 && n_mats <= 65535,
          "transpose_bf16: rows (%d) and cols (%d) must be multiples of 64, n_mats <= 65535", rows, cols);
  REQUIRE(src && dst && src != dst, "transpose_bf16: bad pointers");
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_transpose_rows_bf16(n_mats, rows, cols, src, dst, st), "moe_transpose_bf16", st);
}

moe_status moe_ffn_gate_up_cache_fp8(const moe_shape* shape, int32_t n_experts, int32_t n_rows,
                                     const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                                     const void* a_codes, const float* a_scale, int32_t a_rows, const void* w_gate_up,
                                     const void* w_gu_scale, void* h_codes, float* h_scale, void* gu_codes,
                                     float* gu_scale, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, MOE_F8E4M3, n_experts, n_rows, expert_offsets, 1); r != MOE_OK) return r;
  if (moe_status r = check_gate_up(shape, MOE_F8E4M3, mode, row_src, a_codes, a_scale, a_rows, w_gate_up, w_gu_scale);
      r != MOE_OK)
    return r;
  REQUIRE(h_codes && h_scale && gu_codes && gu_scale, "ffn_gate_up_cache_fp8: h or the cache is NULL");
  SUPPORT(static_cast<long long>(n_rows) * 2 * shape->inter < (1LL << 32),
          "ffn_gate_up_cache_fp8: n_rows * 2 * inter must stay below 2^32");
  if (!workspace || ws_bytes < moe::kFfnQueueBytes)
    return fail(MOE_E_WORKSPACE, "ffn_gate_up_cache_fp8: workspace of %zu bytes < %zu needed", ws_bytes,
                moe::kFfnQueueBytes);
  moe::FfnArgs p{shape->d, shape->inter, n_experts, n_rows, a_rows, expert_offsets, mode, row_src, a_codes, a_scale,
                 w_gate_up, w_gu_scale, nullptr, nullptr, MOE_BF16, nullptr, h_codes, h_scale,
                 static_cast<int*>(workspace)};
  p.gu_cache = gu_codes;
  p.gu_scale = gu_scale;
  auto st = static_cast<hipStream_t>(stream);
  return finish(moe::launch_ffn_fp8_gate_up(p, st), "moe_ffn_gate_up_cache_fp8", st);
}

namespace {
struct Bwd8Layout {
  size_t dyq, dys, dh, dgu, dguq, dgus, h, dyr, hr, dgur, ar, pre, q, total;
};
Bwd8Layout bwd8_layout(const moe_shape* s, int32_t n_rows, int32_t n_experts) {
  const size_t r = static_cast<size_t>(n_rows), d = static_cast<size_t>(s->d), I = static_cast<size_t>(s->inter);
  Bwd8Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  L.dyq = take(r * d);
  L.dys = take(r * (d / 128) * 4);
  L.dh = take(r * I * 4);                             // fp32: the inputs of the quantisers
  L.dgu = take(r * 2 * I * 4);
  L.dguq = take(r * 2 * I);
  L.dgus = take(r * (2 * I / 128) * 4);
  L.h = take(r * I * 4);
  L.dyr = take(r * d * 2);                              // bf16: the re-tiled Wgrad operands (exact E4M3 x 2^k)
  L.hr = take(r * I * 2);
  L.dgur = take(r * 2 * I * 2);
  L.ar = take(r * d * 2);
  L.pre = take((static_cast<size_t>(n_experts) + 1) * 4);
  L.q = take(2 * moe::kFfnQueueBytes);
  L.total = o;
  return L;
}
}  // namespace

size_t moe_ffn_backward_fp8_workspace_bytes(const moe_shape* shape, int32_t n_rows, int32_t n_experts) {
  if (!shape || n_rows < 0 || n_experts <= 0 || shape->d <= 0 || shape->inter <= 0) return 0;
  return bwd8_layout(shape, n_rows, n_experts).total;
}

moe_status moe_ffn_backward_fp8(const moe_shape* shape, int32_t n_experts, int32_t n_rows,
                                const int32_t* expert_offsets, moe_row_mode mode, const int32_t* row_src,
                                const void* a_codes, const float* a_scale, int32_t a_rows, const void* gu_codes,
                                const float* gu_scale, const void* w_gate_up_t, const float* w_gate_up_t_scale,
                                const void* w_down_t, const float* w_down_t_scale, const void* dy, void* da,
                                float* dw_gate_up, float* dw_down, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (moe_status r = check_ffn(shape, MOE_F8E4M3, n_experts, n_rows, expert_offsets, 0); r != MOE_OK) return r;
  REQUIRE(a_codes && a_scale && gu_codes && gu_scale && w_gate_up_t && w_gate_up_t_scale && w_down_t &&
              w_down_t_scale && dy && da && dw_gate_up && dw_down,
          "ffn_backward_fp8: a required pointer is NULL");
  REQUIRE(a_rows > 0, "ffn_backward_fp8: a_rows must be positive");
  REQUIRE(mode == MOE_ROWS_DIRECT || mode == MOE_ROWS_GATHER || mode == MOE_ROWS_SEGMENT,
          "ffn_backward_fp8: bad row mode %d", static_cast<int>(mode));
  REQUIRE(mode != MOE_ROWS_GATHER || row_src != nullptr, "ffn_backward_fp8: MOE_ROWS_GATHER needs row_src");
  const int d = shape->d, I = shape->inter;
  SUPPORT(static_cast<long long>(n_rows) * 2 * I * 4 < (1LL << 32) && static_cast<long long>(n_rows) * d * 2 < (1LL << 32),
          "ffn_backward_fp8: n_rows * 2I must stay below 2^30 and n_rows * d below 2^31 elements");
  SUPPORT(2 * I <= 10240, "ffn_backward_fp8: the input-gradient GEMM of gate/up needs 2 * inter <= 10240");
  const Bwd8Layout L = bwd8_layout(shape, n_rows, n_experts);
  if (!workspace || ws_bytes < L.total)
    return fail(MOE_E_WORKSPACE, "ffn_backward_fp8: workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t o) { return static_cast<void*>(ws + o); };
  float* dys = reinterpret_cast<float*>(ws + L.dys);
  float* dgus = reinterpret_cast<float*>(ws + L.dgus);
  int* pre = reinterpret_cast<int*>(ws + L.pre);
  int* q = reinterpret_cast<int*>(ws + L.q);
  auto st = static_cast<hipStream_t>(stream);
  // Dgrad of the down projection: dh = Q(dy) W_d, dy quantised per 1x128 tile along d
  hipError_t e = moe::launch_quantize_rows(n_rows, d, dy, false, at(L.dyq), dys, st);
  moe::FfnArgs p1{I, d, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, nullptr, nullptr,
                  nullptr, nullptr, w_down_t, w_down_t_scale, MOE_F32, at(L.dh), at(L.dyq), dys, q};
  if (e == hipSuccess) e = moe::launch_ffn_fp8_down(p1, st);
  // SwiGLU backward from the cached E4M3 [G, U]; h recomputed
  if (e == hipSuccess) e = moe::launch_swiglu_backward8(n_rows, I, at(L.dh), gu_codes, gu_scale, at(L.dgu), at(L.h), st);
  // Dgrad of gate/up: da = Q([dG, dU]) W_gate_up
  if (e == hipSuccess) e = moe::launch_quantize_rows(n_rows, 2 * I, at(L.dgu), true, at(L.dguq), dgus, st);
  moe::FfnArgs p2{d, 2 * I, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, nullptr, nullptr,
                  nullptr, nullptr, w_gate_up_t, w_gate_up_t_scale, MOE_BF16, da, at(L.dguq), dgus,
                  q + moe::kQueueInts};
  if (e == hipSuccess) e = moe::launch_ffn_fp8_down(p2, st);
  // Wgrad operands re-tiled to 128x1 (power-of-two scales): dy, h and [dG, dU] by row, a from its 1x128 codes
  if (e == hipSuccess) e = moe::launch_row_block_prefix(n_experts, n_rows, expert_offsets, pre, st);
  if (e == hipSuccess)
    e = moe::launch_requant_cols(d, n_experts, n_rows, expert_offsets, pre, MOE_ROWS_DIRECT, nullptr, n_rows, dy, false,
                                 nullptr, nullptr, at(L.dyr), st);
  if (e == hipSuccess)
    e = moe::launch_requant_cols(I, n_experts, n_rows, expert_offsets, pre, MOE_ROWS_DIRECT, nullptr, n_rows, at(L.h),
                                 true, nullptr, nullptr, at(L.hr), st);
  if (e == hipSuccess)
    e = moe::launch_requant_cols(2 * I, n_experts, n_rows, expert_offsets, pre, MOE_ROWS_DIRECT, nullptr, n_rows,
                                 at(L.dgu), true, nullptr, nullptr, at(L.dgur), st);
  if (e == hipSuccess)
    e = moe::launch_requant_cols(d, n_experts, n_rows, expert_offsets, pre, mode, row_src, a_rows, nullptr, false,
                                 a_codes, a_scale, at(L.ar), st);
  // Wgrad: dW_d = R(dy)^T R(h), dW_gate_up = R([dG, dU])^T R(a)
  if (e == hipSuccess)
    e = moe::launch_wgrad(d, I, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, at(L.dyr),
                          at(L.hr), dw_down, st);
  if (e == hipSuccess)
    e = moe::launch_wgrad(2 * I, d, n_experts, n_rows, n_rows, expert_offsets, MOE_ROWS_DIRECT, nullptr, at(L.dgur),
                          at(L.ar), dw_gate_up, st);
  return finish(e, "moe_ffn_backward_fp8", st);
}


}  // extern "C"
