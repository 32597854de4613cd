// libmoe C ABI: argument validation (on the host, before any HIP call) and
// dispatch to the kernel launchers.  Declarations and the contract of every
// call are in include/libmoe.h.
#include "libmoe.h"
#include "moe_common.h"

#include <rocprofiler-sdk-roctx/roctx.h>

#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <string>

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int64_t kMaxRows = (int64_t)1 << 28;

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status hip_result(hipError_t err, const char* call) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", call, (int)err, hipGetErrorString(err));
}

int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int elem_size(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

// Validation helpers: each returns MOE_OK or records a message naming the argument.
#define MOE_CHECK(expr)                 \
  do {                                  \
    moe_status _st = (expr);            \
    if (_st != MOE_OK) return _st;      \
  } while (0)

moe_status need_ptr(const void* p, const char* fn, const char* name) {
  return p ? MOE_OK : fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s must not be NULL", fn, name);
}

moe_status need_pos(int64_t v, const char* fn, const char* name) {
  return v >= 1 ? MOE_OK : fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s must be >= 1 (got %lld)", fn, name, (long long)v);
}

moe_status need_dtype(moe_dtype dt, const char* fn) {
  return (dt == MOE_F32 || dt == MOE_BF16) ? MOE_OK
                                          : fail(MOE_ERR_INVALID_ARGUMENT, "%s: dt must be MOE_F32 or MOE_BF16 (got %d)",
                                                 fn, (int)dt);
}

moe_status need_layout(moe_weight_layout wl, const char* fn) {
  return (wl == MOE_W_KN || wl == MOE_W_NK)
             ? MOE_OK
             : fail(MOE_ERR_INVALID_ARGUMENT, "%s: weight layout must be MOE_W_KN or MOE_W_NK (got %d)", fn, (int)wl);
}

moe_status need_mult8(int64_t v, const char* fn, const char* name) {
  return v % 8 == 0 ? MOE_OK
                    : fail(MOE_ERR_UNSUPPORTED, "%s: %s must be a multiple of 8 (got %lld)", fn, name, (long long)v);
}

moe_status need_experts(int64_t E, const char* fn) {
  MOE_CHECK(need_pos(E, fn, "E"));
  return E <= moe::kMaxExperts ? MOE_OK
                               : fail(MOE_ERR_UNSUPPORTED, "%s: E must be <= %d (got %lld)", fn, moe::kMaxExperts,
                                      (long long)E);
}

moe_status need_topk(int64_t k, const char* fn) {
  if (k < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: top_k must be positive (got %lld)", fn, (long long)k);
  return k <= moe::kMaxTopK ? MOE_OK
                            : fail(MOE_ERR_UNSUPPORTED, "%s: top_k must be <= %d (got %lld)", fn, moe::kMaxTopK,
                                   (long long)k);
}

moe_status need_rows(int64_t rows, const char* fn, const char* what) {
  return rows < kMaxRows ? MOE_OK
                         : fail(MOE_ERR_UNSUPPORTED, "%s: %s must be < 2^28 (got %lld)", fn, what, (long long)rows);
}

moe_status need_flag(int32_t v, const char* fn, const char* name) {
  return (v == 0 || v == 1) ? MOE_OK
                            : fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s must be 0 or 1 (got %d)", fn, name, (int)v);
}


// Stage of every call, in the stage vocabulary of the PLENA pages
// (PLENA_Compiler PR #69, sections "Group B" and "Group E"; PLENA_Simulator
// PR #97, section "Stage attribution"); '+' joins the stages of a call that
// serves several.  The routed SwiGLU runs in the fc1 epilogue, so it bills to
// expert_projection; the combine overwrites its output, so no separate
// accumulator_init launch exists.  Backward calls carry a "backward:" prefix.
struct CallStage {
  const char* call;
  const char* stage;
};
constexpr CallStage kCallStages[] = {
    {"moe_route", "router_topk"},
    {"moe_route_and_scatter", "router_topk+gather"},
    {"moe_route_and_scatter_noalloc", "router_topk+gather"},
    {"moe_build_scatter", "gather"},
    {"moe_grouped_swiglu_fc1", "expert_projection"},
    {"moe_grouped_fc2", "expert_projection"},
    {"moe_gather_combine", "scatter_combine"},
    {"moe_shared_expert", "shared_expert_projection"},
    {"moe_shared_expert:gated", "shared_expert_gate+shared_expert_projection"},
    {"moe_grouped_swiglu_fc1_mx8", "expert_projection"},
    {"moe_grouped_fc2_mx8", "expert_projection"},
    {"moe_shared_expert_mx8", "shared_expert_projection"},
    {"moe_shared_expert_mx8:gated", "shared_expert_gate+shared_expert_projection"},
    {"moe_grouped_swiglu_fc1_and_shared_mx8", "expert_projection+shared_expert_projection"},
    {"moe_grouped_fc2_and_shared_mx8", "expert_projection+shared_expert_projection"},
    {"moe_grouped_fc2_and_shared_mx8:gated", "expert_projection+shared_expert_gate+shared_expert_projection"},
    {"moe_grouped_swiglu_fc1_and_shared", "expert_projection+shared_expert_projection"},
    {"moe_grouped_swiglu_fc1_gather", "expert_projection"},
    {"moe_grouped_swiglu_fc1_and_shared_gather", "expert_projection+shared_expert_projection"},
    {"moe_grouped_fc2_and_shared", "expert_projection+shared_expert_projection"},
    {"moe_grouped_fc2_and_shared:gated", "expert_projection+shared_expert_gate+shared_expert_projection"},
    {"moe_grouped_swiglu_fc1_save", "expert_projection"},
    {"moe_scatter_grad", "backward:scatter_combine"},
    {"moe_grouped_fc2_backward", "backward:expert_projection"},
    {"moe_grouped_fc1_backward", "backward:expert_projection+backward:gather"},
};

const char* stage_of(const char* call) {
  for (const CallStage& c : kCallStages)
    if (strcmp(c.call, call) == 0) return c.stage;
  return "other";
}

// roctx range around one call, named with its stage: a rocprofv3 marker
// trace then attributes every launch to a stage.
struct StageRange {
  explicit StageRange(const char* stage) { roctxRangePushA(stage); }
  ~StageRange() { roctxRangePop(); }
  StageRange(const StageRange&) = delete;
  StageRange& operator=(const StageRange&) = delete;
};

}  // namespace

extern "C" {

const char* moe_status_name(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_STATUS_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_version(void) { return kVersion; }

const char* moe_call_stage(const char* call, int32_t gated) {
  if (!call) return "other";
  if (gated) {
    const std::string g = std::string(call) + ":gated";
    for (const CallStage& c : kCallStages)
      if (g == c.call) return c.stage;
  }
  return stage_of(call);
}

size_t moe_route_workspace_bytes(moe_dtype dt, int32_t T, int32_t H, int32_t E) {
  if (T < 1 || H < 1 || E < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  return moe_launch::route_workspace_bytes((int)dt, T, H, E);
}

moe_status moe_route(moe_dtype dt, const void* x, const void* w_router, const float* logit_bias, int32_t T, int32_t H,
                     int32_t E, int32_t top_k, int32_t* topk_ids, float* topk_weights, float* logits, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const char* fn = "moe_route";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(w_router, fn, "w_router"));
  MOE_CHECK(need_ptr(topk_ids, fn, "topk_ids"));
  MOE_CHECK(need_ptr(topk_weights, fn, "topk_weights"));
  MOE_CHECK(need_ptr(logits, fn, "logits"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_topk(top_k, fn));
  if (top_k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_route: top_k (%d) exceeds E (%d)", top_k, E);
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_rows((int64_t)T * top_k, fn, "T*top_k"));
  MOE_CHECK(need_rows((int64_t)T * E / 8, fn, "T*E/8"));
  const size_t need = moe_launch::route_workspace_bytes((int)dt, T, H, E);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "moe_route: workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  return hip_result(moe_launch::route((int)dt, x, w_router, logit_bias, T, H, E, top_k, topk_ids, topk_weights, logits,
                                      workspace, (hipStream_t)stream),
                    fn);
}

size_t moe_route_and_scatter_workspace_bytes(moe_dtype dt, int32_t T, int32_t H, int32_t E, int32_t top_k) {
  if (T < 1 || H < 1 || E < 1 || top_k < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  const size_t r = moe_launch::route_workspace_bytes((int)dt, T, H, E);
  const size_t sc = moe_launch::scatter_workspace_bytes(T, top_k, E);
  return r > sc ? r : sc;
}

}  // extern "C"

namespace {

// Argument checks of moe_route_and_scatter and its no-allocation variant
// (everything but the workspace).
moe_status check_route_and_scatter(const char* fn, moe_dtype dt, const void* x, const void* w_router, int32_t T,
                                   int32_t H, int32_t E, int32_t top_k, const int32_t* topk_ids,
                                   const float* topk_weights, const float* logits, const int32_t* scatter_index,
                                   const int32_t* row_token, const int32_t* expert_offsets,
                                   const int32_t* status_words) {
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(w_router, fn, "w_router"));
  MOE_CHECK(need_ptr(topk_ids, fn, "topk_ids"));
  MOE_CHECK(need_ptr(topk_weights, fn, "topk_weights"));
  MOE_CHECK(need_ptr(logits, fn, "logits"));
  MOE_CHECK(need_ptr(scatter_index, fn, "scatter_index"));
  MOE_CHECK(need_ptr(row_token, fn, "row_token"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(status_words, fn, "status_words"));
  // x_scattered may be NULL: the rows are then not copied (the *_gather fc1 calls read x instead)
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_topk(top_k, fn));
  if (top_k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: top_k (%d) exceeds E (%d)", fn, top_k, E);
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_rows((int64_t)T * top_k, fn, "T*top_k"));
  MOE_CHECK(need_rows((int64_t)T * E / 8, fn, "T*E/8"));
  return MOE_OK;
}

// The kernels of moe_route_and_scatter on a validated call, with `workspace`
// holding at least moe_route_and_scatter_workspace_bytes bytes.
moe_status run_route_and_scatter(const char* fn, moe_dtype dt, const void* x, const void* w_router,
                                 const float* logit_bias, int32_t T, int32_t H, int32_t E, int32_t top_k,
                                 int32_t* topk_ids, float* topk_weights, float* logits, int32_t* scatter_index,
                                 int32_t* row_token, int32_t* expert_offsets, int32_t* status_words,
                                 void* x_scattered, void* workspace, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  if (moe_launch::router_small((int)dt, T, E) && moe_launch::route_scatter_fusable(T, top_k, E)) {
    int nsplit = 0;
    hipError_t err = moe_launch::route_partials_small(x, w_router, T, H, E, workspace, &nsplit, s);
    if (err == hipSuccess)
      err = moe_launch::route_scatter_fused((int)dt, (const float*)workspace, nsplit, logit_bias, logits, T, H, E,
                                            top_k, topk_ids, topk_weights, x, scatter_index, row_token,
                                            expert_offsets, status_words, x_scattered, s);
    return hip_result(err, fn);
  }
  hipError_t err = moe_launch::route((int)dt, x, w_router, logit_bias, T, H, E, top_k, topk_ids, topk_weights,
                                     logits, workspace, s);
  if (err == hipSuccess)
    err = moe_launch::build_scatter((int)dt, x, topk_ids, T, H, E, top_k, scatter_index, row_token, expert_offsets,
                                    status_words, x_scattered, workspace, s);
  return hip_result(err, fn);
}

// Scratch of the no-allocation entry point: one array per GPU, allocated
// when the code object loads and held until the process ends.  Host code
// must not pass `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in scratch_addr.
constexpr size_t kScratchBytes = (size_t)64 << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_addr[64] = {};

moe_status scratch_address(const char* fn, void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_result(err, fn);
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "%s: device ordinal %d is beyond 63", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_result(err, fn);
    if (!p) return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress returned no address for the scratch array", fn);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_route_and_scatter(moe_dtype dt, const void* x, const void* w_router, const float* logit_bias,
                                 int32_t T, int32_t H, int32_t E, int32_t top_k, int32_t* topk_ids,
                                 float* topk_weights, float* logits, int32_t* scatter_index, int32_t* row_token,
                                 int32_t* expert_offsets, int32_t* status_words, void* x_scattered, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "moe_route_and_scatter";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(check_route_and_scatter(fn, dt, x, w_router, T, H, E, top_k, topk_ids, topk_weights, logits,
                                    scatter_index, row_token, expert_offsets, status_words));
  const size_t need = moe_route_and_scatter_workspace_bytes(dt, T, H, E, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu%s)", fn, need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  return run_route_and_scatter(fn, dt, x, w_router, logit_bias, T, H, E, top_k, topk_ids, topk_weights, logits,
                               scatter_index, row_token, expert_offsets, status_words, x_scattered, workspace,
                               stream);
}

size_t moe_route_and_scatter_noalloc_max_bytes(void) { return kScratchBytes; }

moe_status moe_route_and_scatter_noalloc(moe_dtype dt, const void* x, const void* w_router, const float* logit_bias,
                                         int32_t T, int32_t H, int32_t E, int32_t top_k, int32_t* topk_ids,
                                         float* topk_weights, float* logits, int32_t* scatter_index,
                                         int32_t* row_token, int32_t* expert_offsets, int32_t* status_words,
                                         void* x_scattered, void* stream) {
  const char* fn = "moe_route_and_scatter_noalloc";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(check_route_and_scatter(fn, dt, x, w_router, T, H, E, top_k, topk_ids, topk_weights, logits,
                                    scatter_index, row_token, expert_offsets, status_words));
  const size_t need = moe_route_and_scatter_workspace_bytes(dt, T, H, E, top_k);
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "%s: these sizes need %zu bytes of scratch, more than the %zu bytes the "
                "library holds per device (use moe_route_and_scatter with a workspace)", fn, need, kScratchBytes);
  void* ws = nullptr;
  MOE_CHECK(scratch_address(fn, &ws));
  return run_route_and_scatter(fn, dt, x, w_router, logit_bias, T, H, E, top_k, topk_ids, topk_weights, logits,
                               scatter_index, row_token, expert_offsets, status_words, x_scattered, ws, stream);
}

size_t moe_build_scatter_workspace_bytes(int32_t T, int32_t top_k, int32_t E) {
  if (T < 1 || top_k < 1 || E < 1) return 0;
  return moe_launch::scatter_workspace_bytes(T, top_k, E);
}

moe_status moe_build_scatter(moe_dtype dt, const void* x, const int32_t* topk_ids, int32_t T, int32_t H, int32_t E,
                             int32_t top_k, int32_t* scatter_index, int32_t* row_token, int32_t* expert_offsets,
                             int32_t* status_words, void* x_scattered, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const char* fn = "moe_build_scatter";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(topk_ids, fn, "topk_ids"));
  MOE_CHECK(need_ptr(scatter_index, fn, "scatter_index"));
  MOE_CHECK(need_ptr(row_token, fn, "row_token"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(status_words, fn, "status_words"));
  // x_scattered may be NULL: the rows are then not copied (the *_gather fc1 calls read x instead)
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_topk(top_k, fn));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_rows((int64_t)T * top_k, fn, "T*top_k"));
  const size_t need = moe_launch::scatter_workspace_bytes(T, top_k, E);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_build_scatter: workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  return hip_result(moe_launch::build_scatter((int)dt, x, topk_ids, T, H, E, top_k, scatter_index, row_token,
                                              expert_offsets, status_words, x_scattered, workspace,
                                              (hipStream_t)stream),
                    fn);
}

moe_status moe_grouped_swiglu_fc1(moe_dtype dt, moe_weight_layout wl, const void* x_scattered,
                                  const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H, int32_t E,
                                  int32_t I, void* act, void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(x_scattered, fn, "x_scattered"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1, fn, "w1"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  return hip_result(moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x_scattered, expert_offsets, E, R, w1,
                                                   (int64_t)H * 2 * I, H, I, act, 0, cu_count(), (hipStream_t)stream),
                    fn);
}

moe_status moe_grouped_fc2(moe_dtype dt, moe_weight_layout wl, const void* act, const int32_t* expert_offsets,
                           const void* w2, int32_t R, int32_t I, int32_t E, int32_t H, float* y_rows, void* stream) {
  const char* fn = "moe_grouped_fc2";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w2, fn, "w2"));
  MOE_CHECK(need_ptr(y_rows, fn, "y_rows"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  return hip_result(moe_launch::grouped_fc2((int)dt, (int)wl, act, expert_offsets, E, R, w2, (int64_t)I * H, I, H,
                                            y_rows, nullptr, 0, 1, 0, cu_count(), (hipStream_t)stream),
                    fn);
}

moe_status moe_gather_combine(const float* y_rows, const int32_t* scatter_index, const float* topk_weights, int32_t T,
                              int32_t H, int32_t top_k, int32_t accumulate, float* y, void* stream) {
  const char* fn = "moe_gather_combine";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_ptr(y_rows, fn, "y_rows"));
  MOE_CHECK(need_ptr(scatter_index, fn, "scatter_index"));
  MOE_CHECK(need_ptr(topk_weights, fn, "topk_weights"));
  MOE_CHECK(need_ptr(y, fn, "y"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_topk(top_k, fn));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_flag(accumulate, fn, "accumulate"));
  MOE_CHECK(need_rows((int64_t)T * top_k, fn, "T*top_k"));
  return hip_result(moe_launch::gather_combine(y_rows, scatter_index, topk_weights, T, H, top_k, accumulate, y,
                                               (hipStream_t)stream),
                    fn);
}

size_t moe_shared_expert_workspace_bytes(moe_dtype dt, int32_t T, int32_t I_s) {
  if (T < 1 || I_s < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  return align256((size_t)T * I_s * elem_size(dt)) + align256((size_t)T * sizeof(float));
}

moe_status moe_shared_expert(moe_dtype dt, moe_weight_layout wl, const void* x, const void* ws1, const void* ws2,
                             const void* w_gate, int32_t T, int32_t H, int32_t I_s, int32_t accumulate, float* y,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_shared_expert";
  StageRange stage_range(stage_of(w_gate ? "moe_shared_expert:gated" : fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(ws1, fn, "ws1"));
  MOE_CHECK(need_ptr(ws2, fn, "ws2"));
  MOE_CHECK(need_ptr(y, fn, "y"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I_s, fn, "I_s"));
  MOE_CHECK(need_flag(accumulate, fn, "accumulate"));
  MOE_CHECK(need_rows(T, fn, "T"));
  const size_t need = moe_shared_expert_workspace_bytes(dt, T, I_s);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_shared_expert: workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* act = ws;
  float* gate = w_gate ? (float*)(ws + align256((size_t)T * I_s * elem_size(dt))) : nullptr;
  const int cus = cu_count();
  if (gate) MOE_CHECK(hip_result(moe_launch::shared_gate((int)dt, x, w_gate, T, H, gate, s), fn));
  MOE_CHECK(hip_result(
      moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x, nullptr, 1, T, ws1, 0, H, I_s, act, 1, cus, s), fn));
  return hip_result(
      moe_launch::grouped_fc2((int)dt, (int)wl, act, nullptr, 1, T, ws2, 0, I_s, H, y, gate, accumulate, 0, 1, cus, s),
      fn);
}

moe_status need_mult128(int64_t v, const char* fn, const char* name) {
  return v % 128 == 0 ? MOE_OK
                      : fail(MOE_ERR_UNSUPPORTED, "%s: %s must be a multiple of 128 for MXFP8 weights (got %lld)", fn,
                             name, (long long)v);
}

moe_status moe_grouped_swiglu_fc1_mx8(const void* x_scattered, const int32_t* expert_offsets, const uint8_t* w1q,
                                      const uint8_t* w1s, int32_t R, int32_t H, int32_t E, int32_t I, void* act,
                                      void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1_mx8";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_ptr(x_scattered, fn, "x_scattered"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1q, fn, "w1q"));
  MOE_CHECK(need_ptr(w1s, fn, "w1s"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_mult128(H, fn, "H"));
  MOE_CHECK(need_rows(R, fn, "R"));
  return hip_result(moe_launch::grouped_swiglu_fc1_mx8(x_scattered, expert_offsets, E, R, w1q, w1s, H, I, act, 0,
                                                       cu_count(), (hipStream_t)stream),
                    fn);
}

moe_status moe_grouped_fc2_mx8(const void* act, const int32_t* expert_offsets, const uint8_t* w2q,
                               const uint8_t* w2s, int32_t R, int32_t I, int32_t E, int32_t H, float* y_rows,
                               void* stream) {
  const char* fn = "moe_grouped_fc2_mx8";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w2q, fn, "w2q"));
  MOE_CHECK(need_ptr(w2s, fn, "w2s"));
  MOE_CHECK(need_ptr(y_rows, fn, "y_rows"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult128(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  return hip_result(moe_launch::grouped_fc2_mx8(act, expert_offsets, E, R, w2q, w2s, I, H, y_rows, nullptr, 0, 1, 0,
                                                cu_count(), (hipStream_t)stream),
                    fn);
}

moe_status moe_shared_expert_mx8(const void* x, const uint8_t* ws1q, const uint8_t* ws1s, const uint8_t* ws2q,
                                 const uint8_t* ws2s, const void* w_gate, int32_t T, int32_t H, int32_t I_s,
                                 int32_t accumulate, float* y, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const char* fn = "moe_shared_expert_mx8";
  StageRange stage_range(stage_of(w_gate ? "moe_shared_expert_mx8:gated" : fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(ws1q, fn, "ws1q"));
  MOE_CHECK(need_ptr(ws1s, fn, "ws1s"));
  MOE_CHECK(need_ptr(ws2q, fn, "ws2q"));
  MOE_CHECK(need_ptr(ws2s, fn, "ws2s"));
  MOE_CHECK(need_ptr(y, fn, "y"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult128(H, fn, "H"));
  MOE_CHECK(need_mult128(I_s, fn, "I_s"));
  MOE_CHECK(need_flag(accumulate, fn, "accumulate"));
  MOE_CHECK(need_rows(T, fn, "T"));
  const size_t need = moe_shared_expert_workspace_bytes(MOE_BF16, T, I_s);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu%s)", fn, need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* act = ws;
  float* gate = w_gate ? (float*)(ws + align256((size_t)T * I_s * elem_size(MOE_BF16))) : nullptr;
  const int cus = cu_count();
  if (gate) MOE_CHECK(hip_result(moe_launch::shared_gate(1, x, w_gate, T, H, gate, s), fn));
  MOE_CHECK(hip_result(moe_launch::grouped_swiglu_fc1_mx8(x, nullptr, 1, T, ws1q, ws1s, H, I_s, act, 1, cus, s), fn));
  return hip_result(moe_launch::grouped_fc2_mx8(act, nullptr, 1, T, ws2q, ws2s, I_s, H, y, gate, accumulate, 0, 1, cus,
                                                s),
                    fn);
}

moe_status moe_grouped_swiglu_fc1_and_shared_mx8(const void* x_scattered, const int32_t* expert_offsets,
                                                 const uint8_t* w1q, const uint8_t* w1s, int32_t R, int32_t H,
                                                 int32_t E, int32_t I, void* act, const void* x, const uint8_t* ws1q,
                                                 const uint8_t* ws1s, int32_t T, int32_t I_s, void* act_shared,
                                                 void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1_and_shared_mx8";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_ptr(x_scattered, fn, "x_scattered"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1q, fn, "w1q"));
  MOE_CHECK(need_ptr(w1s, fn, "w1s"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(ws1q, fn, "ws1q"));
  MOE_CHECK(need_ptr(ws1s, fn, "ws1s"));
  MOE_CHECK(need_ptr(act_shared, fn, "act_shared"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult128(H, fn, "H"));
  MOE_CHECK(need_mult128(I, fn, "I"));
  MOE_CHECK(need_mult128(I_s, fn, "I_s"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows(T, fn, "T"));
  return hip_result(moe_launch::fused_fc1_mx8(x_scattered, expert_offsets, E, R, w1q, w1s, H, I, act, x, T, ws1q,
                                              ws1s, I_s, act_shared, cu_count(), (hipStream_t)stream),
                    fn);
}

moe_status moe_grouped_fc2_and_shared_mx8(const void* act, const int32_t* expert_offsets, const uint8_t* w2q,
                                          const uint8_t* w2s, int32_t R, int32_t I, int32_t E, int32_t H,
                                          float* y_rows, const void* act_shared, const uint8_t* ws2q,
                                          const uint8_t* ws2s, const void* x, const void* w_gate, int32_t T,
                                          int32_t I_s, int32_t accumulate, float* y, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  const char* fn = "moe_grouped_fc2_and_shared_mx8";
  StageRange stage_range(stage_of(w_gate ? "moe_grouped_fc2_and_shared_mx8:gated" : fn));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w2q, fn, "w2q"));
  MOE_CHECK(need_ptr(w2s, fn, "w2s"));
  MOE_CHECK(need_ptr(y_rows, fn, "y_rows"));
  MOE_CHECK(need_ptr(act_shared, fn, "act_shared"));
  MOE_CHECK(need_ptr(ws2q, fn, "ws2q"));
  MOE_CHECK(need_ptr(ws2s, fn, "ws2s"));
  MOE_CHECK(need_ptr(y, fn, "y"));
  if (w_gate) MOE_CHECK(need_ptr(x, fn, "x (needed for the gate)"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult128(I, fn, "I"));
  MOE_CHECK(need_mult128(I_s, fn, "I_s"));
  MOE_CHECK(need_flag(accumulate, fn, "accumulate"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows(T, fn, "T"));
  const size_t need = moe_shared_expert_workspace_bytes(MOE_BF16, T, I_s);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu%s)", fn, need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  float* gate = w_gate ? (float*)((char*)workspace + align256((size_t)T * I_s * elem_size(MOE_BF16))) : nullptr;
  if (gate) MOE_CHECK(hip_result(moe_launch::shared_gate(1, x, w_gate, T, H, gate, s), fn));
  return hip_result(moe_launch::fused_fc2_mx8(act, expert_offsets, E, R, w2q, w2s, I, H, y_rows, act_shared, T, ws2q,
                                              ws2s, I_s, gate, accumulate, y, cu_count(), s),
                    fn);
}

int32_t moe_grouped_gemm_tile(moe_dtype dt, int32_t call, int32_t R, int32_t H, int32_t E, int32_t I, int32_t T,
                              int32_t I_s) {
  if ((dt != MOE_F32 && dt != MOE_BF16) || (call != 0 && call != 1) || R < 1 || H < 1 || E < 1 || I < 1 ||
      E > moe::kMaxExperts || I_s < 0 || (I_s > 0 && T < 1))
    return -1;
  return moe_launch::tile_config((int)dt, call, R, H, E, I, T, I_s, cu_count());
}

int32_t moe_and_shared_launches(moe_dtype dt, int32_t R, int32_t H, int32_t E, int32_t I, int32_t T, int32_t I_s) {
  if (R < 1 || H < 1 || E < 1 || I < 1 || T < 1 || I_s < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  return moe_launch::fused_supported((int)dt, H, I, I_s, E, R, T) ? 1 : 2;
}

moe_status moe_grouped_swiglu_fc1_and_shared(moe_dtype dt, moe_weight_layout wl, const void* x_scattered,
                                             const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H,
                                             int32_t E, int32_t I, void* act, const void* x, const void* ws1,
                                             int32_t T, int32_t I_s, void* act_shared, void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1_and_shared";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(x_scattered, fn, "x_scattered"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1, fn, "w1"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(ws1, fn, "ws1"));
  MOE_CHECK(need_ptr(act_shared, fn, "act_shared"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_mult8(I_s, fn, "I_s"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows(T, fn, "T"));
  hipStream_t s = (hipStream_t)stream;
  const int cus = cu_count();
  if (moe_launch::fused_supported((int)dt, H, I, I_s, E, R, T))
    return hip_result(moe_launch::fused_fc1((int)wl, x_scattered, expert_offsets, E, R, w1, H, I, act, x, T, ws1,
                                            I_s, act_shared, cus, s),
                      fn);
  MOE_CHECK(hip_result(moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x_scattered, expert_offsets, E, R, w1,
                                                      (int64_t)H * 2 * I, H, I, act, 0, cus, s),
                       fn));
  return hip_result(
      moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x, nullptr, 1, T, ws1, 0, H, I_s, act_shared, 1, cus, s), fn);
}

moe_status moe_grouped_swiglu_fc1_gather(moe_dtype dt, moe_weight_layout wl, const void* x, const int32_t* row_token,
                                         const int32_t* expert_offsets, const void* w1, int32_t T, int32_t R,
                                         int32_t H, int32_t E, int32_t I, void* act, void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1_gather";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(row_token, fn, "row_token"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1, fn, "w1"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows(T, fn, "T"));
  return hip_result(moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x, expert_offsets, E, R, w1, (int64_t)H * 2 * I,
                                                   H, I, act, 0, cu_count(), (hipStream_t)stream, row_token, T),
                    fn);
}

moe_status moe_grouped_swiglu_fc1_and_shared_gather(moe_dtype dt, moe_weight_layout wl, const void* x,
                                                    const int32_t* row_token, const int32_t* expert_offsets,
                                                    const void* w1, int32_t R, int32_t H, int32_t E, int32_t I,
                                                    void* act, const void* ws1, int32_t T, int32_t I_s,
                                                    void* act_shared, void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1_and_shared_gather";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(x, fn, "x"));
  MOE_CHECK(need_ptr(row_token, fn, "row_token"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1, fn, "w1"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(ws1, fn, "ws1"));
  MOE_CHECK(need_ptr(act_shared, fn, "act_shared"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_mult8(I_s, fn, "I_s"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows(T, fn, "T"));
  hipStream_t s = (hipStream_t)stream;
  const int cus = cu_count();
  if (moe_launch::fused_supported((int)dt, H, I, I_s, E, R, T))
    return hip_result(moe_launch::fused_fc1((int)wl, x, expert_offsets, E, R, w1, H, I, act, x, T, ws1, I_s,
                                            act_shared, cus, s, row_token),
                      fn);
  MOE_CHECK(hip_result(moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x, expert_offsets, E, R, w1,
                                                      (int64_t)H * 2 * I, H, I, act, 0, cus, s, row_token, T),
                       fn));
  return hip_result(
      moe_launch::grouped_swiglu_fc1((int)dt, (int)wl, x, nullptr, 1, T, ws1, 0, H, I_s, act_shared, 1, cus, s), fn);
}

moe_status moe_grouped_fc2_and_shared(moe_dtype dt, moe_weight_layout wl, const void* act,
                                      const int32_t* expert_offsets, const void* w2, int32_t R, int32_t I, int32_t E,
                                      int32_t H, float* y_rows, const void* act_shared, const void* ws2,
                                      const void* x, const void* w_gate, int32_t T, int32_t I_s, int32_t accumulate,
                                      float* y, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_grouped_fc2_and_shared";
  StageRange stage_range(stage_of(w_gate ? "moe_grouped_fc2_and_shared:gated" : fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w2, fn, "w2"));
  MOE_CHECK(need_ptr(y_rows, fn, "y_rows"));
  MOE_CHECK(need_ptr(act_shared, fn, "act_shared"));
  MOE_CHECK(need_ptr(ws2, fn, "ws2"));
  MOE_CHECK(need_ptr(y, fn, "y"));
  if (w_gate) MOE_CHECK(need_ptr(x, fn, "x (needed for the gate)"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(I_s, fn, "I_s"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_mult8(I_s, fn, "I_s"));
  MOE_CHECK(need_flag(accumulate, fn, "accumulate"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows(T, fn, "T"));
  const size_t need = moe_shared_expert_workspace_bytes(dt, T, I_s);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_fc2_and_shared: workspace needs %zu bytes (got %zu%s)", need,
                workspace_bytes, workspace ? "" : ", NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  float* gate = w_gate ? (float*)((char*)workspace + align256((size_t)T * I_s * elem_size(dt))) : nullptr;
  const int cus = cu_count();
  if (gate) MOE_CHECK(hip_result(moe_launch::shared_gate((int)dt, x, w_gate, T, H, gate, s), fn));
  if (moe_launch::fused_supported((int)dt, H, I, I_s, E, R, T))
    return hip_result(moe_launch::fused_fc2((int)wl, act, expert_offsets, E, R, w2, I, H, y_rows, act_shared, T,
                                            ws2, I_s, gate, accumulate, y, cus, s),
                      fn);
  MOE_CHECK(hip_result(moe_launch::grouped_fc2((int)dt, (int)wl, act, expert_offsets, E, R, w2, (int64_t)I * H, I, H,
                                               y_rows, nullptr, 0, 1, 0, cus, s),
                       fn));
  return hip_result(moe_launch::grouped_fc2((int)dt, (int)wl, act_shared, nullptr, 1, T, ws2, 0, I_s, H, y, gate,
                                            accumulate, 0, 1, cus, s),
                    fn);
}

// ------------------------------------------------------------------------------------------
// Backward of the routed experts
// ------------------------------------------------------------------------------------------
moe_status moe_grouped_swiglu_fc1_save(moe_dtype dt, moe_weight_layout wl, const void* x_scattered,
                                       const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H,
                                       int32_t E, int32_t I, void* act, void* h_pre, void* stream) {
  const char* fn = "moe_grouped_swiglu_fc1_save";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(x_scattered, fn, "x_scattered"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1, fn, "w1"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(h_pre, fn, "h_pre"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  return hip_result(moe_launch::grouped_swiglu_fc1_save((int)dt, (int)wl, x_scattered, expert_offsets, E, R, w1,
                                                        (int64_t)H * 2 * I, H, I, act, h_pre, cu_count(),
                                                        (hipStream_t)stream),
                    fn);
}

moe_status moe_scatter_grad(moe_dtype dt, const float* dy, const float* y_rows, const float* topk_weights,
                            const int32_t* scatter_index, int32_t T, int32_t H, int32_t top_k, int32_t R,
                            void* d_rows, float* d_topk_weights, void* stream) {
  const char* fn = "moe_scatter_grad";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_ptr(dy, fn, "dy"));
  MOE_CHECK(need_ptr(y_rows, fn, "y_rows"));
  MOE_CHECK(need_ptr(topk_weights, fn, "topk_weights"));
  MOE_CHECK(need_ptr(scatter_index, fn, "scatter_index"));
  MOE_CHECK(need_ptr(d_rows, fn, "d_rows"));
  MOE_CHECK(need_ptr(d_topk_weights, fn, "d_topk_weights"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_topk(top_k, fn));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_rows((int64_t)T * top_k, fn, "T*top_k"));
  MOE_CHECK(need_rows(R, fn, "R"));
  return hip_result(moe_launch::scatter_grad((int)dt, dy, y_rows, topk_weights, scatter_index, T, H, top_k, R, d_rows,
                                             d_topk_weights, (hipStream_t)stream),
                    fn);
}

moe_status moe_grouped_fc2_backward(moe_dtype dt, moe_weight_layout wl, const void* d_rows, const void* act,
                                    const void* h_pre, const int32_t* expert_offsets, const void* w2, int32_t R,
                                    int32_t I, int32_t E, int32_t H, void* d_h, void* d_w2, void* stream) {
  const char* fn = "moe_grouped_fc2_backward";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(d_rows, fn, "d_rows"));
  MOE_CHECK(need_ptr(act, fn, "act"));
  MOE_CHECK(need_ptr(h_pre, fn, "h_pre"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w2, fn, "w2"));
  MOE_CHECK(need_ptr(d_h, fn, "d_h"));
  MOE_CHECK(need_ptr(d_w2, fn, "d_w2"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  const hipStream_t s = (hipStream_t)stream;
  const int cus = cu_count();
  hipError_t err = moe_launch::grouped_fc2_dgrad_swiglu((int)dt, (int)wl, d_rows, expert_offsets, E, R, w2, I, H,
                                                        h_pre, d_h, cus, s);
  // d_w2 in the layout of w2: [I, H] = act^T d_rows, or [H, I] = d_rows^T act.
  if (err == hipSuccess)
    err = wl == MOE_W_KN ? moe_launch::grouped_wgrad((int)dt, act, d_rows, expert_offsets, E, R, I, H, d_w2, 2, cus, s)
                         : moe_launch::grouped_wgrad((int)dt, d_rows, act, expert_offsets, E, R, H, I, d_w2, 2, cus, s);
  return hip_result(err, fn);
}

size_t moe_grouped_fc1_backward_workspace_bytes(int32_t R, int32_t H) {
  if (R < 1 || H < 1) return 0;
  return align256((size_t)R * H * sizeof(float));
}

moe_status moe_grouped_fc1_backward(moe_dtype dt, moe_weight_layout wl, const void* d_h, const void* x_scattered,
                                    const int32_t* expert_offsets, const void* w1, int32_t R, int32_t H, int32_t E,
                                    int32_t I, const int32_t* scatter_index, int32_t T, int32_t top_k,
                                    int32_t accumulate, float* d_x, void* d_w1, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const char* fn = "moe_grouped_fc1_backward";
  StageRange stage_range(stage_of(fn));
  MOE_CHECK(need_dtype(dt, fn));
  MOE_CHECK(need_layout(wl, fn));
  MOE_CHECK(need_ptr(d_h, fn, "d_h"));
  MOE_CHECK(need_ptr(x_scattered, fn, "x_scattered"));
  MOE_CHECK(need_ptr(expert_offsets, fn, "expert_offsets"));
  MOE_CHECK(need_ptr(w1, fn, "w1"));
  MOE_CHECK(need_ptr(scatter_index, fn, "scatter_index"));
  MOE_CHECK(need_ptr(d_x, fn, "d_x"));
  MOE_CHECK(need_ptr(d_w1, fn, "d_w1"));
  MOE_CHECK(need_pos(R, fn, "R"));
  MOE_CHECK(need_pos(H, fn, "H"));
  MOE_CHECK(need_experts(E, fn));
  MOE_CHECK(need_pos(I, fn, "I"));
  MOE_CHECK(need_pos(T, fn, "T"));
  MOE_CHECK(need_topk(top_k, fn));
  MOE_CHECK(need_flag(accumulate, fn, "accumulate"));
  MOE_CHECK(need_mult8(H, fn, "H"));
  MOE_CHECK(need_mult8(I, fn, "I"));
  MOE_CHECK(need_rows(R, fn, "R"));
  MOE_CHECK(need_rows((int64_t)T * top_k, fn, "T*top_k"));
  const size_t need = moe_grouped_fc1_backward_workspace_bytes(R, H);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu%s)", fn, need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  const hipStream_t s = (hipStream_t)stream;
  const int cus = cu_count();
  float* d_xs = (float*)workspace;
  hipError_t err = moe_launch::grouped_fc1_dgrad((int)dt, (int)wl, d_h, expert_offsets, E, R, w1, H, I, d_xs, cus, s);
  if (err == hipSuccess)
    err = moe_launch::gather_combine(d_xs, scatter_index, nullptr, T, H, top_k, accumulate, d_x, s);
  // d_w1 in the layout of w1: [H, 2I] = x_scattered^T d_h, or [2I, H] = d_h^T x_scattered.
  if (err == hipSuccess)
    err = wl == MOE_W_KN
              ? moe_launch::grouped_wgrad((int)dt, x_scattered, d_h, expert_offsets, E, R, H, 2 * I, d_w1, 1, cus, s)
              : moe_launch::grouped_wgrad((int)dt, d_h, x_scattered, expert_offsets, E, R, 2 * I, H, d_w1, 1, cus, s);
  return hip_result(err, fn);
}

}  // extern "C"
