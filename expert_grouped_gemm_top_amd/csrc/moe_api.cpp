// moe_api.cpp -- the C ABI of libmoe (declared in include/moe.h): argument
// validation, then the kernel launches on the caller's stream.  Validation runs
// before anything is enqueued, so a rejected call leaves the stream untouched.
// No C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "moe.h"
#include "moe_launch.h"

namespace moe {
namespace {
thread_local int64_t g_launches = 0;  // kernel launches made from this thread
}  // namespace
void note_launch() { ++g_launches; }
thread_local LaunchEvents g_launch_events;
LaunchEvents& launch_events() { return g_launch_events; }
}  // namespace moe

namespace {

thread_local std::string g_last_error;

// one-shot event pairs armed by moe_profile_kernel, per kernel kind
struct Armed {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local Armed g_armed[MOE_K_COUNT];
// one-shot event armed by moe_signal_dh_ready; the next dx call takes it
thread_local hipEvent_t g_dh_ready = nullptr;

hipError_t record_if(hipEvent_t ev, hipStream_t s) { return ev == nullptr ? hipSuccess : hipEventRecord(ev, s); }

// Runs one kernel launch `f` (returning hipError_t) between the armed events of `kind`.
// The phase's launches record the events in their own dispatch (MOE_LAUNCH);
// a phase that launched nothing records both here, an empty interval.
template <typename Fn>
hipError_t timed(int kind, hipStream_t s, Fn&& f) {
  Armed& a = g_armed[kind];
  if (a.start == nullptr) return f();
  moe::LaunchEvents& ev = moe::launch_events();
  ev.start = a.start;
  ev.stop = a.stop;
  hipError_t err = f();
  const bool launched = ev.start == nullptr;
  ev = moe::LaunchEvents{};
  if (err == hipSuccess && !launched) err = hipEventRecord(a.start, s);
  if (err == hipSuccess && !launched) err = hipEventRecord(a.stop, s);
  a = Armed{};
  return err;
}

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t err, const char* where) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(err), (int)err);
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int esize_of(int dtype) { return dtype == MOE_F32 ? 4 : (dtype == MOE_BF16 ? 2 : 0); }

#define REQUIRE(cond, status, ...)        \
  do {                                    \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)
#define NONNULL(p) REQUIRE((p) != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: %s must not be NULL", fn, #p)

int check_routing_dims(const char* fn, int T, int E, int k) {
  REQUIRE(T >= 1 && E >= 1 && k >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: T=%d, E=%d, k=%d must be >= 1", fn, T, E, k);
  REQUIRE(k <= E, MOE_ERR_INVALID_ARGUMENT, "%s: k=%d exceeds E=%d", fn, k, E);
  REQUIRE(E <= moe::kMaxExpertsHost, MOE_ERR_UNSUPPORTED, "%s: E=%d exceeds 256", fn, E);
  REQUIRE(k <= 16, MOE_ERR_UNSUPPORTED, "%s: k=%d exceeds 16", fn, k);
  REQUIRE((int64_t)T * k < (int64_t)1 << 31, MOE_ERR_UNSUPPORTED, "%s: T*k=%lld reaches 2^31", fn,
          (long long)T * k);
  return MOE_OK;
}

int check_dtype(const char* fn, int dtype) {
  REQUIRE(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_INVALID_ARGUMENT, "%s: dtype %d is neither MOE_F32 nor MOE_BF16",
          fn, dtype);
  return MOE_OK;
}

int check_row_width(const char* fn, const char* name, int v) {
  REQUIRE(v >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: %s=%d must be >= 1", fn, name, v);
  REQUIRE(v % 8 == 0, MOE_ERR_UNSUPPORTED, "%s: %s=%d is not a multiple of 8", fn, name, v);
  return MOE_OK;
}

// An optional row map (rows gathered on load): its divisor when present.
int check_row_map(const char* fn, const char* name, const int32_t* map, int div) {
  if (map != nullptr)
    REQUIRE(div >= 1 && div <= 16, MOE_ERR_INVALID_ARGUMENT, "%s: %s divisor %d must be in 1..16", fn, name, div);
  return MOE_OK;
}

int check_expert_dims(const char* fn, int H, int F, int E, int dtype) {
  int rc = check_dtype(fn, dtype);
  if (rc) return rc;
  if ((rc = check_row_width(fn, "H", H)) || (rc = check_row_width(fn, "F", F))) return rc;
  REQUIRE(E >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: E=%d must be >= 1", fn, E);
  REQUIRE(E <= moe::kMaxExpertsHost, MOE_ERR_UNSUPPORTED, "%s: E=%d exceeds 256", fn, E);
  REQUIRE((int64_t)E * H * F < ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "%s: weights too large", fn);
  return MOE_OK;
}

const int kGemmKind[4] = {MOE_K_GEMM_GATEUP, MOE_K_GEMM_DOWN, MOE_K_GEMM_DA, MOE_K_GEMM_DX};

int check_rows(const char* fn, int max_rows) {
  REQUIRE(max_rows >= 0, MOE_ERR_INVALID_ARGUMENT, "%s: max_rows=%d is negative", fn, max_rows);
  return MOE_OK;
}

int check_router_workspace(const char* fn, int T, int H, int E, const void* ws, size_t ws_bytes) {
  const size_t need = moe::router_workspace_bytes(T, H, E);
  REQUIRE(ws_bytes >= need, MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  REQUIRE(need == 0 || ws != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: workspace must not be NULL", fn);
  REQUIRE(((uintptr_t)ws & 15) == 0, MOE_ERR_INVALID_ARGUMENT, "%s: workspace must be 16-byte aligned", fn);
  return MOE_OK;
}

// The expert forward; with perm, row s of the gate/up product reads
// x[perm[s] / k] (gathered on load) instead of x_sorted[s].
// s_gu / s_down non-NULL: the weights are fp8 (E4M3) with those per-expert scales.
int swiglu_fwd(const char* fn, int H, int F, int E, int max_rows, int max_expert_rows, int dtype, const int32_t* offsets,
               const void* x_rows, const int32_t* perm, int k, const void* w_gate, const void* w_up, const void* w_down,
               void* h_save, void* a_save, void* o_sorted, void* stream, const float* s_gu = nullptr,
               const float* s_down = nullptr) {
  const bool w8 = s_gu != nullptr;
  int rc = check_expert_dims(fn, H, F, E, dtype);
  if (rc || (rc = check_rows(fn, max_rows))) return rc;
  REQUIRE(max_expert_rows >= 0, MOE_ERR_INVALID_ARGUMENT, "%s: max_expert_rows=%d is negative", fn, max_expert_rows);
  NONNULL(offsets);
  REQUIRE(x_rows != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: %s must not be NULL", fn, perm ? "x" : "x_sorted");
  NONNULL(w_gate);
  NONNULL(w_up);
  NONNULL(w_down);
  NONNULL(a_save);
  NONNULL(o_sorted);
  if (max_rows == 0) return MOE_OK;
  moe::RowGemmArgs g{};
  g.offsets = offsets;
  g.E = E;
  g.H = H;
  g.F = F;
  hipStream_t s = as_stream(stream);
  auto run = [&](int mode) {
    return timed(kGemmKind[mode], s, [&] {
      if (w8) return moe::launch_row_gemm_fp8w(mode, g, max_rows, s);
      return dtype == MOE_BF16 ? moe::launch_row_gemm_bf16(mode, g, max_rows, max_expert_rows, s)
                               : moe::launch_row_gemm_f32(mode, g, max_rows, s);
    });
  };
  g.a = (const uint16_t*)x_rows;
  g.a_map = perm;
  g.a_div = k;
  g.w0 = (const uint16_t*)w_gate;
  g.w1 = (const uint16_t*)w_up;
  g.out0 = (uint16_t*)h_save;
  g.out1 = (uint16_t*)a_save;
  g.wscale = s_gu;
  if ((rc = hip_status(run(moe::kGemmGateUp), fn))) return rc;
  g.a = (const uint16_t*)a_save;
  g.a_map = nullptr;
  g.a_div = 1;
  g.w0 = (const uint16_t*)w_down;
  g.w1 = nullptr;
  g.out0 = (uint16_t*)o_sorted;
  g.out1 = nullptr;
  g.wscale = s_down;
  return hip_status(run(moe::kGemmDown), fn);
}

// fp8 weights of one call: present, 8-byte aligned (the kernels load 8 bytes at
// a time), scales present.
int check_fp8_weights(const char* fn, const void* wq_gate, const void* wq_up, const void* wq_down, const float* s_gu,
                      const float* s_down) {
  NONNULL(wq_gate);
  NONNULL(wq_up);
  NONNULL(wq_down);
  NONNULL(s_gu);
  NONNULL(s_down);
  REQUIRE(((uintptr_t)wq_gate | (uintptr_t)wq_up | (uintptr_t)wq_down) % 8 == 0, MOE_ERR_INVALID_ARGUMENT,
          "%s: fp8 weights must be 8-byte aligned", fn);
  return MOE_OK;
}

int bwd_dx(const char* fn, int T, int H, int F, int E, int k, int max_rows, int dtype, const int32_t* offsets,
           const int32_t* inv, const void* dy, const float* topk_w, const void* h_rows, const int32_t* h_src,
           const void* w_gate,
           const void* w_up, const void* w_down, const int32_t* inv_all, const void* o_sorted, float* dg,
           void* dO_rows, void* dh_rows, void* dX_rows, void* dx, void* stream, const float* s_gu,
           const float* s_down) {
  const bool w8 = s_gu != nullptr;
  const hipEvent_t dh_ready = g_dh_ready;  // taken by this call whatever its outcome
  g_dh_ready = nullptr;
  int rc = check_routing_dims(fn, T, E, k);
  if (rc || (rc = check_expert_dims(fn, H, F, E, dtype)) || (rc = check_rows(fn, max_rows))) return rc;
  REQUIRE(max_rows <= T * k, MOE_ERR_INVALID_ARGUMENT, "%s: max_rows=%d exceeds T*k=%d", fn, max_rows, T * k);
  NONNULL(offsets);
  NONNULL(inv);
  NONNULL(dy);
  NONNULL(topk_w);
  NONNULL(h_rows);
  NONNULL(w_gate);
  NONNULL(w_up);
  NONNULL(w_down);
  NONNULL(dO_rows);
  NONNULL(dh_rows);
  NONNULL(dX_rows);
  NONNULL(dx);
  if (dg != nullptr) {
    NONNULL(inv_all);
    NONNULL(o_sorted);
  }
  hipStream_t s = as_stream(stream);
  const int es = esize_of(dtype);
  if ((rc = hip_status(timed(MOE_K_GRAD_ROWS, s,
                             [&] {
                               return moe::launch_grad_rows(T, H, k, es, dy, topk_w, inv, dO_rows, inv_all, o_sorted,
                                                            dg, s);
                             }),
                       fn)))
    return rc;
  if (max_rows > 0) {
    moe::RowGemmArgs g{};
    g.offsets = offsets;
    g.E = E;
    g.H = H;
    g.F = F;
    auto run = [&](int mode) {
      return timed(kGemmKind[mode], s, [&] {
        // rows of one expert come from distinct pairs of distinct tokens when
        // the routing picks distinct experts per token: T bounds them
        if (w8) return moe::launch_row_gemm_fp8w(mode, g, max_rows, s);
        return dtype == MOE_BF16 ? moe::launch_row_gemm_bf16(mode, g, max_rows, std::min(max_rows, T), s)
                                 : moe::launch_row_gemm_f32(mode, g, max_rows, s);
      });
    };
    g.a = (const uint16_t*)dO_rows;
    g.w0 = (const uint16_t*)w_down;
    g.h = (const uint16_t*)h_rows;
    g.h_map = h_src;
    g.out0 = (uint16_t*)dh_rows;
    g.wscale = s_down;
    if ((rc = hip_status(run(moe::kGemmDA), fn))) return rc;
    if ((rc = hip_status(record_if(dh_ready, s), fn))) return rc;
    g.a = (const uint16_t*)dh_rows;
    g.w0 = (const uint16_t*)w_gate;
    g.w1 = (const uint16_t*)w_up;
    g.h = nullptr;
    g.h_map = nullptr;
    g.out0 = (uint16_t*)dX_rows;
    g.wscale = s_gu;
    if ((rc = hip_status(run(moe::kGemmDX), fn))) return rc;
  } else if ((rc = hip_status(record_if(dh_ready, s), fn))) {  // no rows: dO (and dg) are all there is
    return rc;
  }
  return hip_status(timed(MOE_K_COMBINE, s, [&] { return moe::launch_combine(T, H, k, es, dX_rows, inv, nullptr, dx, s); }),
                    fn);
}

int check_dispatch(const char* fn, int T, int H, int E, int k, int dtype, const int32_t* topk_idx, const void* x,
                   const int32_t* counts, const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                   const void* x_sorted) {
  int rc = check_routing_dims(fn, T, E, k);
  if (rc) return rc;
  if ((rc = check_dtype(fn, dtype)) || (rc = check_row_width(fn, "H", H))) return rc;
  NONNULL(topk_idx);
  NONNULL(counts);
  NONNULL(offsets);
  NONNULL(perm);
  NONNULL(inv_perm);
  REQUIRE((x == nullptr) == (x_sorted == nullptr), MOE_ERR_INVALID_ARGUMENT,
          "%s: x and x_sorted must both be given or both be NULL", fn);
  return MOE_OK;
}

// The dispatch kernels with workspace `ws` (at least dispatch_workspace_bytes).
int dispatch_launch(const char* fn, int T, int H, int E, int k, int dtype, const int32_t* topk_idx, const void* x,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_sorted, void* ws,
                    hipStream_t s) {
  int rc;
  if ((rc = hip_status(moe::launch_dispatch_index(T, E, k, topk_idx, counts, offsets, perm, inv_perm, ws, s), fn)))
    return rc;
  if (x_sorted == nullptr) return MOE_OK;
  return hip_status(timed(MOE_K_DISPATCH_ROWS, s,
                          [&] { return moe::launch_dispatch_rows(T, H, k, esize_of(dtype), x, inv_perm, x_sorted, s); }),
                    fn);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_abi_version(void) { return 8; }

int64_t moe_launch_count(void) { return moe::g_launches; }

int moe_profile_kernel(int kernel, void* start_event, void* stop_event) {
  const char* fn = "moe_profile_kernel";
  REQUIRE(kernel >= 0 && kernel < MOE_K_COUNT, MOE_ERR_INVALID_ARGUMENT, "%s: unknown kernel %d", fn, kernel);
  REQUIRE((start_event == nullptr) == (stop_event == nullptr), MOE_ERR_INVALID_ARGUMENT,
          "%s: give both events or neither", fn);
  g_armed[kernel].start = reinterpret_cast<hipEvent_t>(start_event);
  g_armed[kernel].stop = reinterpret_cast<hipEvent_t>(stop_event);
  return MOE_OK;
}

int moe_signal_dh_ready(void* event) {
  g_dh_ready = reinterpret_cast<hipEvent_t>(event);
  return MOE_OK;
}

size_t moe_router_workspace_bytes(int T, int H, int E) {
  if (T < 1 || H < 1 || E < 1) return 0;
  return moe::router_workspace_bytes(T, H, E);
}

int moe_router_fwd(int T, int H, int E, int dtype, const void* x, const void* w_r, float* logits, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const char* fn = "moe_router_fwd";
  int rc = check_routing_dims(fn, T, E, 1);
  if (rc || (rc = check_dtype(fn, dtype)) || (rc = check_row_width(fn, "H", H))) return rc;
  REQUIRE((int64_t)T * H < ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "%s: x too large", fn);
  NONNULL(x);
  NONNULL(w_r);
  NONNULL(logits);
  if ((rc = check_router_workspace(fn, T, H, E, workspace, workspace_bytes))) return rc;
  hipStream_t s = as_stream(stream);
  return hip_status(timed(MOE_K_ROUTER_FWD, s,
                          [&] { return moe::launch_router_fwd(T, H, E, esize_of(dtype), x, w_r, logits, workspace, s); }),
                    fn);
}

int moe_route_topk(int T, int E, int k, const float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  const char* fn = "moe_route_topk";
  int rc = check_routing_dims(fn, T, E, k);
  if (rc) return rc;
  NONNULL(logits);
  NONNULL(topk_idx);
  NONNULL(topk_w);
  hipStream_t s = as_stream(stream);
  return hip_status(timed(MOE_K_ROUTE, s, [&] { return moe::launch_route_topk(T, E, k, logits, topk_idx, topk_w, s); }), fn);
}

size_t moe_dispatch_workspace_bytes(int T, int E, int k) {
  if (T < 1 || E < 1 || k < 1) return 0;
  return moe::dispatch_workspace_bytes((int64_t)T * k, E);
}

int moe_dispatch(int T, int H, int E, int k, int dtype, const int32_t* topk_idx, const void* x, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_sorted, void* workspace,
                 size_t workspace_bytes, void* stream) {
  const char* fn = "moe_dispatch";
  int rc = check_dispatch(fn, T, H, E, k, dtype, topk_idx, x, counts, offsets, perm, inv_perm, x_sorted);
  if (rc) return rc;
  const size_t need = moe::dispatch_workspace_bytes((int64_t)T * k, E);
  REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", fn,
          workspace_bytes, need);
  REQUIRE(need == 0 || workspace != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: workspace must not be NULL", fn);
  return dispatch_launch(fn, T, H, E, k, dtype, topk_idx, x, counts, offsets, perm, inv_perm, x_sorted, workspace,
                         as_stream(stream));
}

size_t moe_dispatch_noalloc_max_workspace(void) { return moe::kDispatchScratchBytes; }

int moe_dispatch_noalloc(int T, int H, int E, int k, int dtype, const int32_t* topk_idx, const void* x,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_sorted,
                         void* stream) {
  const char* fn = "moe_dispatch_noalloc";
  int rc = check_dispatch(fn, T, H, E, k, dtype, topk_idx, x, counts, offsets, perm, inv_perm, x_sorted);
  if (rc) return rc;
  const size_t need = moe::dispatch_workspace_bytes((int64_t)T * k, E);
  REQUIRE(need <= moe::kDispatchScratchBytes, MOE_ERR_UNSUPPORTED,
          "%s: T=%d, E=%d, k=%d need %zu bytes of workspace, above the library's %zu (use moe_dispatch with a "
          "caller workspace)",
          fn, T, E, k, need, moe::kDispatchScratchBytes);
  void* ws = nullptr;
  if (need > 0 && (rc = hip_status(moe::dispatch_scratch(&ws), fn))) return rc;
  return dispatch_launch(fn, T, H, E, k, dtype, topk_idx, x, counts, offsets, perm, inv_perm, x_sorted, ws,
                         as_stream(stream));
}

int moe_grouped_swiglu_fwd(int H, int F, int E, int max_rows, int max_expert_rows, int dtype, const int32_t* offsets,
                           const void* x_sorted, const void* w_gate, const void* w_up, const void* w_down, void* h_save,
                           void* a_save, void* o_sorted, void* stream) {
  return swiglu_fwd("moe_grouped_swiglu_fwd", H, F, E, max_rows, max_expert_rows, dtype, offsets, x_sorted, nullptr, 1,
                    w_gate, w_up, w_down, h_save, a_save, o_sorted, stream);
}

int moe_grouped_swiglu_fwd_fp8w(int H, int F, int E, int k, int max_rows, const int32_t* offsets, const void* x_rows,
                                const int32_t* perm, const uint8_t* wq_gate, const uint8_t* wq_up,
                                const uint8_t* wq_down, const float* s_gu, const float* s_down, void* h_save,
                                void* a_save, void* o_sorted, void* stream) {
  const char* fn = "moe_grouped_swiglu_fwd_fp8w";
  REQUIRE(perm == nullptr || (k >= 1 && k <= 16), MOE_ERR_INVALID_ARGUMENT, "%s: k=%d must be in 1..16", fn, k);
  const int rc = check_fp8_weights(fn, wq_gate, wq_up, wq_down, s_gu, s_down);
  if (rc) return rc;
  return swiglu_fwd(fn, H, F, E, max_rows, max_rows, MOE_BF16, offsets, x_rows, perm, perm ? k : 1, wq_gate, wq_up,
                    wq_down, h_save, a_save, o_sorted, stream, s_gu, s_down);
}

int moe_quantize_weights_fp8(int E, int64_t n0, int64_t n1, const void* w0, const void* w1, uint8_t* q0, uint8_t* q1,
                             float* scale, void* stream) {
  const char* fn = "moe_quantize_weights_fp8";
  REQUIRE(E >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: E=%d must be >= 1", fn, E);
  REQUIRE(n0 >= 8 && n0 % 8 == 0, MOE_ERR_UNSUPPORTED, "%s: n0=%lld must be a positive multiple of 8", fn,
          (long long)n0);
  NONNULL(w0);
  NONNULL(q0);
  NONNULL(scale);
  REQUIRE((w1 == nullptr) == (q1 == nullptr), MOE_ERR_INVALID_ARGUMENT, "%s: w1 and q1 must both be given or both be NULL",
          fn);
  if (w1 != nullptr)
    REQUIRE(n1 >= 8 && n1 % 8 == 0, MOE_ERR_UNSUPPORTED, "%s: n1=%lld must be a positive multiple of 8", fn,
            (long long)n1);
  else
    REQUIRE(n1 == 0, MOE_ERR_INVALID_ARGUMENT, "%s: n1=%lld must be 0 without w1", fn, (long long)n1);
  REQUIRE(((uintptr_t)w0 | (uintptr_t)w1) % 16 == 0 && ((uintptr_t)q0 | (uintptr_t)q1) % 8 == 0,
          MOE_ERR_INVALID_ARGUMENT, "%s: w0/w1 must be 16-byte and q0/q1 8-byte aligned", fn);
  REQUIRE((int64_t)E * (n0 > n1 ? n0 : n1) < ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "%s: matrices too large", fn);
  hipStream_t s = as_stream(stream);
  return hip_status(moe::launch_quantize_fp8(E, n0, n1, (const uint16_t*)w0, (const uint16_t*)w1, q0, q1, scale, s),
                    fn);
}

int moe_quantize_rows_fp8(int rows, int cols, const void* x, uint8_t* q, float* scale, void* stream) {
  const char* fn = "moe_quantize_rows_fp8";
  REQUIRE(rows >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: rows=%d must be >= 1", fn, rows);
  REQUIRE(cols >= 8 && cols % 8 == 0, MOE_ERR_UNSUPPORTED, "%s: cols=%d must be a positive multiple of 8", fn, cols);
  NONNULL(x);
  NONNULL(q);
  NONNULL(scale);
  REQUIRE((uintptr_t)x % 16 == 0 && (uintptr_t)q % 8 == 0, MOE_ERR_INVALID_ARGUMENT,
          "%s: x must be 16-byte and q 8-byte aligned", fn);
  REQUIRE((int64_t)rows * cols < ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "%s: matrix too large", fn);
  return hip_status(moe::launch_quantize_rows_fp8(rows, cols, (const uint16_t*)x, q, scale, as_stream(stream)), fn);
}

int moe_transpose_fp8(int E, int rows, int cols, const uint8_t* in, uint8_t* out, void* stream) {
  const char* fn = "moe_transpose_fp8";
  REQUIRE(E >= 1 && rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: E=%d, rows=%d, cols=%d must be >= 1", fn, E,
          rows, cols);
  REQUIRE(rows % 16 == 0 && cols % 16 == 0, MOE_ERR_UNSUPPORTED, "%s: rows=%d and cols=%d must be multiples of 16", fn,
          rows, cols);
  REQUIRE(rows <= (1 << 24) && cols <= (1 << 24) && E <= 65535, MOE_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  NONNULL(in);
  NONNULL(out);
  REQUIRE(in != out, MOE_ERR_INVALID_ARGUMENT, "%s: in and out must not be the same buffer", fn);
  REQUIRE(((uintptr_t)in | (uintptr_t)out) % 16 == 0, MOE_ERR_INVALID_ARGUMENT, "%s: in and out must be 16-byte aligned",
          fn);
  return hip_status(moe::launch_transpose_u8(E, rows, cols, in, out, as_stream(stream)), fn);
}

int moe_grouped_swiglu_fwd_fp8(int H, int F, int E, int k, int max_rows, const int32_t* offsets, const uint8_t* xq,
                               const float* x_scale, const int32_t* perm, const uint8_t* wt_gate,
                               const uint8_t* wt_up, const uint8_t* wt_down, const float* s_gu, const float* s_down,
                               void* h_save, void* a_save, uint8_t* aq, float* a_scale, void* o_sorted,
                               void* stream) {
  const char* fn = "moe_grouped_swiglu_fwd_fp8";
  int rc = check_expert_dims(fn, H, F, E, MOE_BF16);
  if (rc || (rc = check_rows(fn, max_rows))) return rc;
  REQUIRE(H % 16 == 0 && F % 16 == 0, MOE_ERR_UNSUPPORTED, "%s: H=%d and F=%d must be multiples of 16", fn, H, F);
  REQUIRE(perm == nullptr || (k >= 1 && k <= 16), MOE_ERR_INVALID_ARGUMENT, "%s: k=%d must be in 1..16", fn, k);
  NONNULL(offsets);
  NONNULL(xq);
  NONNULL(x_scale);
  NONNULL(wt_gate);
  NONNULL(wt_up);
  NONNULL(wt_down);
  NONNULL(s_gu);
  NONNULL(s_down);
  NONNULL(a_save);
  NONNULL(aq);
  NONNULL(a_scale);
  NONNULL(o_sorted);
  REQUIRE(((uintptr_t)xq | (uintptr_t)wt_gate | (uintptr_t)wt_up | (uintptr_t)wt_down | (uintptr_t)aq |
           (uintptr_t)a_save) % 16 == 0,
          MOE_ERR_INVALID_ARGUMENT, "%s: codes and a_save must be 16-byte aligned", fn);
  if (max_rows == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  moe::Fp8GemmArgs g{};
  g.offsets = offsets;
  g.E = E;
  g.H = H;
  g.F = F;
  g.a = xq;
  g.a_map = perm;
  g.a_div = perm ? k : 1;
  g.ascale = x_scale;
  g.w0 = wt_gate;
  g.w1 = wt_up;
  g.wscale = s_gu;
  g.out0 = (uint16_t*)h_save;
  g.out1 = (uint16_t*)a_save;
  if ((rc = hip_status(timed(MOE_K_GEMM_GATEUP, s, [&] { return moe::launch_gemm_fp8(moe::kGemmGateUp, g, max_rows, s); }),
                       fn)))
    return rc;
  // the stored SwiGLU output, one power-of-two scale per row, for the down product
  if ((rc = hip_status(moe::launch_quantize_rows_fp8(max_rows, F, (const uint16_t*)a_save, aq, a_scale, s),
                       fn)))
    return rc;
  g.a = aq;
  g.a_map = nullptr;
  g.a_div = 1;
  g.ascale = a_scale;
  g.w0 = wt_down;
  g.w1 = nullptr;
  g.wscale = s_down;
  g.out0 = (uint16_t*)o_sorted;
  g.out1 = nullptr;
  return hip_status(timed(MOE_K_GEMM_DOWN, s, [&] { return moe::launch_gemm_fp8(moe::kGemmDown, g, max_rows, s); }), fn);
}

int moe_grouped_swiglu_fwd_gather(int H, int F, int E, int k, int max_rows, int max_expert_rows, int dtype,
                                  const int32_t* offsets, const void* x, const int32_t* perm, const void* w_gate,
                                  const void* w_up, const void* w_down, void* h_save, void* a_save, void* o_sorted,
                                  void* stream) {
  const char* fn = "moe_grouped_swiglu_fwd_gather";
  REQUIRE(k >= 1 && k <= 16, MOE_ERR_INVALID_ARGUMENT, "%s: k=%d must be in 1..16", fn, k);
  NONNULL(perm);
  return swiglu_fwd(fn, H, F, E, max_rows, max_expert_rows, dtype, offsets, x, perm, k, w_gate, w_up, w_down, h_save,
                    a_save, o_sorted, stream);
}

int moe_grouped_swiglu_recompute(int H, int F, int E, int max_rows, int max_expert_rows, int dtype,
                                 const int32_t* offsets, const void* x_rows, const int32_t* x_src, int x_div,
                                 const void* w_gate, const void* w_up, void* h_rows, void* a_rows, void* stream) {
  const char* fn = "moe_grouped_swiglu_recompute";
  int rc = check_expert_dims(fn, H, F, E, dtype);
  if (rc || (rc = check_rows(fn, max_rows)) || (rc = check_row_map(fn, "x_src", x_src, x_div))) return rc;
  REQUIRE(max_expert_rows >= 0, MOE_ERR_INVALID_ARGUMENT, "%s: max_expert_rows=%d is negative", fn, max_expert_rows);
  NONNULL(offsets);
  NONNULL(x_rows);
  NONNULL(w_gate);
  NONNULL(w_up);
  NONNULL(h_rows);
  if (max_rows == 0) return MOE_OK;
  moe::RowGemmArgs g{};
  g.offsets = offsets;
  g.E = E;
  g.H = H;
  g.F = F;
  g.a = (const uint16_t*)x_rows;
  g.a_map = x_src;
  g.a_div = x_src ? x_div : 1;
  g.w0 = (const uint16_t*)w_gate;
  g.w1 = (const uint16_t*)w_up;
  g.out0 = (uint16_t*)h_rows;
  g.out1 = (uint16_t*)a_rows;
  hipStream_t s = as_stream(stream);
  return hip_status(timed(MOE_K_GEMM_GATEUP, s,
                          [&] {
                            return dtype == MOE_BF16
                                       ? moe::launch_row_gemm_bf16(moe::kGemmGateUp, g, max_rows, max_expert_rows, s)
                                       : moe::launch_row_gemm_f32(moe::kGemmGateUp, g, max_rows, s);
                          }),
                    fn);
}

int moe_combine(int T, int H, int k, int dtype, const void* rows, const int32_t* inv, const float* topk_w, void* out,
                void* stream) {
  const char* fn = "moe_combine";
  REQUIRE(T >= 1 && k >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: T=%d, k=%d must be >= 1", fn, T, k);
  REQUIRE(k <= 16, MOE_ERR_UNSUPPORTED, "%s: k=%d exceeds 16", fn, k);
  REQUIRE((int64_t)T * k < (int64_t)1 << 31, MOE_ERR_UNSUPPORTED, "%s: T*k reaches 2^31", fn);
  int rc;
  if ((rc = check_dtype(fn, dtype)) || (rc = check_row_width(fn, "H", H))) return rc;
  NONNULL(rows);
  NONNULL(inv);
  NONNULL(out);
  hipStream_t s = as_stream(stream);
  return hip_status(
      timed(MOE_K_COMBINE, s, [&] { return moe::launch_combine(T, H, k, esize_of(dtype), rows, inv, topk_w, out, s); }),
      fn);
}

int moe_grouped_bwd_dx(int T, int H, int F, int E, int k, int max_rows, int dtype, const int32_t* offsets,
                       const int32_t* inv, const void* dy, const float* topk_w, const void* h_rows,
                       const int32_t* h_src, const void* w_gate, const void* w_up, const void* w_down,
                       const int32_t* inv_all, const void* o_sorted, float* dg, void* dO_rows, void* dh_rows,
                       void* dX_rows, void* dx, void* stream) {
  return bwd_dx("moe_grouped_bwd_dx", T, H, F, E, k, max_rows, dtype, offsets, inv, dy, topk_w, h_rows, h_src, w_gate,
                w_up, w_down, inv_all, o_sorted, dg, dO_rows, dh_rows, dX_rows, dx, stream, nullptr, nullptr);
}

int moe_grouped_bwd_dx_fp8w(int T, int H, int F, int E, int k, int max_rows, const int32_t* offsets,
                            const int32_t* inv, const void* dy, const float* topk_w, const void* h_rows,
                            const int32_t* h_src, const uint8_t* wq_gate, const uint8_t* wq_up, const uint8_t* wq_down, const float* s_gu,
                            const float* s_down, const int32_t* inv_all, const void* o_sorted, float* dg,
                            void* dO_rows, void* dh_rows, void* dX_rows, void* dx, void* stream) {
  const char* fn = "moe_grouped_bwd_dx_fp8w";
  const int rc = check_fp8_weights(fn, wq_gate, wq_up, wq_down, s_gu, s_down);
  if (rc) return rc;
  return bwd_dx(fn, T, H, F, E, k, max_rows, MOE_BF16, offsets, inv, dy, topk_w, h_rows, h_src, wq_gate, wq_up,
                wq_down, inv_all, o_sorted, dg, dO_rows, dh_rows, dX_rows, dx, stream, s_gu, s_down);
}

int moe_grouped_bwd_dw(int H, int F, int E, int max_rows, int dtype, const int32_t* offsets, const void* x_rows,
                       const int32_t* x_src, int x_div, const void* a_rows, const int32_t* a_src,
                       const void* dO_rows, const void* dh_rows, void* dw_gate, void* dw_up, void* dw_down,
                       void* stream) {
  const char* fn = "moe_grouped_bwd_dw";
  int rc = check_expert_dims(fn, H, F, E, dtype);
  if (rc || (rc = check_rows(fn, max_rows)) || (rc = check_row_map(fn, "x_src", x_src, x_div))) return rc;
  NONNULL(offsets);
  NONNULL(dw_gate);
  NONNULL(dw_up);
  NONNULL(dw_down);
  if (max_rows > 0) {
    NONNULL(x_rows);
    NONNULL(a_rows);
    NONNULL(dO_rows);
    NONNULL(dh_rows);
  }
  moe::DwArgs g{};
  g.offsets = offsets;
  g.E = E;
  g.H = H;
  g.F = F;
  g.x = (const uint16_t*)x_rows;
  g.x_map = x_src;
  g.x_div = x_src ? x_div : 1;
  g.a = (const uint16_t*)a_rows;
  g.a_map = a_src;
  g.dO = (const uint16_t*)dO_rows;
  g.dh = (const uint16_t*)dh_rows;
  g.dwg = (uint16_t*)dw_gate;
  g.dwu = (uint16_t*)dw_up;
  g.dwd = (uint16_t*)dw_down;
  hipStream_t s = as_stream(stream);
  return hip_status(
      timed(MOE_K_GEMM_DW, s, [&] { return dtype == MOE_BF16 ? moe::launch_dw_bf16(g, s) : moe::launch_dw_f32(g, s); }),
      fn);
}

int moe_router_bwd(int T, int H, int E, int k, int dtype, const void* x, const void* w_r, const int32_t* topk_idx,
                   const float* topk_w, const float* dg, float* dlogits, void* dw_r, void* dx, int dx_accumulate,
                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_router_bwd";
  int rc = check_routing_dims(fn, T, E, k);
  if (rc || (rc = check_dtype(fn, dtype)) || (rc = check_row_width(fn, "H", H))) return rc;
  REQUIRE((int64_t)T * H < ((int64_t)1 << 40), MOE_ERR_UNSUPPORTED, "%s: x too large", fn);
  NONNULL(x);
  NONNULL(w_r);
  NONNULL(topk_idx);
  NONNULL(topk_w);
  NONNULL(dg);
  NONNULL(dlogits);
  NONNULL(dw_r);
  NONNULL(dx);
  if ((rc = check_router_workspace(fn, T, H, E, workspace, workspace_bytes))) return rc;
  hipStream_t s = as_stream(stream);
  return hip_status(timed(MOE_K_ROUTER_DW, s,
                          [&] {
                            return moe::launch_router_bwd(T, H, E, k, esize_of(dtype), x, w_r, topk_idx, topk_w, dg,
                                                          dlogits, dw_r, dx, dx_accumulate != 0, workspace, s);
                          }),
                    fn);
}

int moe_compact_pairs(int T, int H, int F, int E, int k, int dtype, double rho, const int32_t* counts,
                      const int32_t* offsets, const int32_t* perm, const float* score, int32_t* kept_counts,
                      int32_t* kept_offsets, int32_t* kept_perm, int32_t* kept_src, int32_t* kept_inv,
                      const void* x_sorted, const void* a_save, const void* h_save, void* x_kept, void* a_kept,
                      void* h_kept, void* stream) {
  const char* fn = "moe_compact_pairs";
  REQUIRE(rho > 0.0 && std::isfinite(rho), MOE_ERR_INVALID_ARGUMENT, "%s: rho=%g must be positive and finite", fn,
          rho);
  int rc = check_routing_dims(fn, T, E, k);
  if (rc) return rc;
  const int64_t cap64 = moe_quota_cap(T, E, k, rho);
  return moe_compact_pairs_cap(T, H, F, E, k, dtype, (int)std::min<int64_t>(cap64, (int64_t)T * k), counts, offsets,
                               perm, score, kept_counts, kept_offsets, kept_perm, kept_src, kept_inv, x_sorted, a_save,
                               h_save, x_kept, a_kept, h_kept, stream);
}

int64_t moe_quota_cap_for_budget(int T, int H, int F, int E, int k, int dtype, int with_dw, int keep_graph,
                                 size_t budget_bytes) {
  if (T < 1 || H < 1 || F < 1 || E < 1 || k < 1 || (dtype != MOE_F32 && dtype != MOE_BF16)) return -1;
  const int64_t eb = dtype == MOE_F32 ? 4 : 2;
  const int64_t row_bytes = eb * (3 * (int64_t)H + 2 * (int64_t)F + (keep_graph ? 2 * (int64_t)F : 0) +
                                  (with_dw ? (int64_t)F : 0));
  const int64_t cap = (int64_t)(budget_bytes / (uint64_t)(E * row_bytes));
  if (cap < 1) return -1;
  const int64_t most = ((int64_t)T * k + E - 1) / E;
  return cap < most ? cap : most;
}

int moe_pair_scores(int T, int H, int F, int k, int dtype, const int32_t* inv_perm, const float* topk_w,
                    const void* a_save, const void* dy, float* score, void* stream) {
  const char* fn = "moe_pair_scores";
  REQUIRE(T >= 1 && k >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: T=%d, k=%d must be >= 1", fn, T, k);
  REQUIRE(k <= 16, MOE_ERR_UNSUPPORTED, "%s: k=%d exceeds 16", fn, k);
  REQUIRE((int64_t)T * k < (int64_t)1 << 31, MOE_ERR_UNSUPPORTED, "%s: T*k=%lld reaches 2^31", fn, (long long)T * k);
  int rc;
  if ((rc = check_dtype(fn, dtype)) || (rc = check_row_width(fn, "H", H)) || (rc = check_row_width(fn, "F", F)))
    return rc;
  NONNULL(inv_perm);
  NONNULL(topk_w);
  NONNULL(a_save);
  NONNULL(dy);
  NONNULL(score);
  hipStream_t s = as_stream(stream);
  return hip_status(moe::launch_pair_scores(T, H, F, k, esize_of(dtype), inv_perm, topk_w, a_save, dy, score, s), fn);
}

int64_t moe_quota_cap(int T, int E, int k, double rho) {
  if (T < 1 || E < 1 || k < 1 || !(rho > 0.0) || !std::isfinite(rho)) return -1;
  if (rho == 1.0) return ((int64_t)T * k + E - 1) / E;
  const double c = std::ceil(rho * (double)T * (double)k / (double)E);
  const double n = (double)T * k;
  return (int64_t)(c < n ? c : n);
}

int moe_compact_pairs_cap(int T, int H, int F, int E, int k, int dtype, int cap, const int32_t* counts,
                          const int32_t* offsets, const int32_t* perm, const float* score, int32_t* kept_counts,
                          int32_t* kept_offsets, int32_t* kept_perm, int32_t* kept_src, int32_t* kept_inv,
                          const void* x_sorted, const void* a_save, const void* h_save, void* x_kept, void* a_kept,
                          void* h_kept, void* stream) {
  const char* fn = "moe_compact_pairs_cap";
  int rc = check_routing_dims(fn, T, E, k);
  if (rc || (rc = check_dtype(fn, dtype))) return rc;
  REQUIRE(cap >= 1, MOE_ERR_INVALID_ARGUMENT, "%s: quota cap=%d must be >= 1", fn, cap);
  NONNULL(counts);
  NONNULL(offsets);
  NONNULL(perm);
  NONNULL(score);
  NONNULL(kept_counts);
  NONNULL(kept_offsets);
  NONNULL(kept_perm);
  NONNULL(kept_src);
  NONNULL(kept_inv);
  REQUIRE(x_sorted == nullptr || x_kept != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: x_kept must not be NULL", fn);
  REQUIRE(a_save == nullptr || a_kept != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: a_kept must not be NULL", fn);
  REQUIRE(h_save == nullptr || h_kept != nullptr, MOE_ERR_INVALID_ARGUMENT, "%s: h_kept must not be NULL", fn);
  if (x_sorted && (rc = check_row_width(fn, "H", H))) return rc;
  if ((a_save || h_save) && (rc = check_row_width(fn, "F", F))) return rc;
  const int64_t N = (int64_t)T * k;
  if ((int64_t)cap > N) cap = (int)N;
  hipStream_t s = as_stream(stream);
  if ((rc = hip_status(moe::launch_fill_i32(kept_inv, N, -1, s), fn))) return rc;
  if ((rc = hip_status(timed(MOE_K_COMPACT, s,
                             [&] {
                               return moe::launch_compact(N, E, cap, counts, offsets, perm, score, kept_counts,
                                                          kept_offsets, kept_perm, kept_src, kept_inv, s);
                             }),
                       fn)))
    return rc;
  if (!x_sorted && !a_save && !h_save) return MOE_OK;
  const int64_t bound64 = (int64_t)E * cap < N ? (int64_t)E * cap : N;
  const int es = esize_of(dtype);
  return hip_status(moe::launch_gather_rows(kept_offsets + E, kept_src, (int)bound64, x_sorted, x_kept, H * es, a_save,
                                            a_kept, F * es, h_save, h_kept, 2 * F * es, s),
                    fn);
}

}  // extern "C"
