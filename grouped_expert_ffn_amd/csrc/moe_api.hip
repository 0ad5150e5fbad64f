// The exported C ABI of libmoe (declared in include/moe.h): argument checks, workspace
// layout, and the choice between the decode (grouped GEMV) and prefill (MFMA grouped GEMM)
// kernels.  Every check runs on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "moe_internal.h"

namespace moe {

namespace {

thread_local std::string g_last_error;
thread_local void* g_timer_start[MOE_KERNEL_COUNT];
thread_local void* g_timer_stop[MOE_KERNEL_COUNT];

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int32_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

int32_t device_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxDim = 16384;
constexpr int kMaxTokens = 1 << 20;

// Descriptor checks shared by every call.
int32_t check_desc(const moe_layer_desc_t* d, LayerDims* L) {
  if (!d) return fail(MOE_ERR_INVALID, "desc is NULL");
  if (d->d_model <= 0 || d->d_ff <= 0) return fail(MOE_ERR_INVALID, "d_model and d_ff must be > 0");
  if (d->n_experts < 1) return fail(MOE_ERR_INVALID, "n_experts must be >= 1");
  if (d->top_k < 1 || d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID, "top_k must be in [1, n_experts]");
  if (d->n_shared < 0) return fail(MOE_ERR_INVALID, "n_shared must be >= 0");
  if (d->renormalize != 0 && d->renormalize != 1) return fail(MOE_ERR_INVALID, "renormalize must be 0 or 1");
  if (d->pre_norm != 0 && d->pre_norm != 1) return fail(MOE_ERR_INVALID, "pre_norm must be 0 or 1");
  if (d->pre_norm && !(d->norm_eps >= 0.f && d->norm_eps < 1e30f))
    return fail(MOE_ERR_INVALID, "norm_eps must be finite and >= 0");
  if (!(d->capacity_factor >= 0.f && d->capacity_factor < 1e30f))
    return fail(MOE_ERR_INVALID, "capacity_factor must be finite and >= 0");
  if (d->n_experts > 256) return fail(MOE_ERR_UNSUPPORTED, "n_experts > 256");
  if (d->top_k > 16) return fail(MOE_ERR_UNSUPPORTED, "top_k > 16");
  if (d->n_shared > 8) return fail(MOE_ERR_UNSUPPORTED, "n_shared > 8");
  if (d->d_model % 16 || d->d_ff % 16)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 16");
  if (d->d_model > kMaxDim || d->d_ff > kMaxDim)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be <= %d", kMaxDim);
  const bool combo = (d->act_dtype == MOE_F32 && d->w_dtype == MOE_F32) ||
                     (d->act_dtype == MOE_BF16 && d->w_dtype == MOE_BF16) ||
                     (d->act_dtype == MOE_BF16 && d->w_dtype == MOE_I8);
  if (!combo)
    return fail(MOE_ERR_UNSUPPORTED, "dtype combination act=%d w=%d (supported: f32/f32, bf16/bf16, bf16/i8)",
                d->act_dtype, d->w_dtype);
  *L = LayerDims{d->d_model, d->n_experts, d->top_k, d->d_ff, d->n_shared, d->renormalize,
                 d->act_dtype, d->w_dtype, d->capacity_factor};
  return MOE_OK;
}

int32_t check_tokens(const LayerDims& L, int32_t T) {
  if (T < 0) return fail(MOE_ERR_INVALID, "T must be >= 0");
  if (T > kMaxTokens) return fail(MOE_ERR_UNSUPPORTED, "T > %d", kMaxTokens);
  if ((int64_t)T * (L.k + L.S) > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "T*(k+S) > 2^24");
  return MOE_OK;
}

#define REQUIRE_PTR(p)                                                      \
  do {                                                                      \
    if (!(p)) return fail(MOE_ERR_INVALID, "%s is NULL", #p);               \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID, "%s is not 16-byte aligned", #p); \
  } while (0)
#define CHECK_ALIGN(p)                                                      \
  do {                                                                      \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_INVALID, "%s is not 16-byte aligned", #p); \
  } while (0)

size_t esz(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }
size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

// moe_forward workspace sections
struct FwdLayout {
  size_t xn, logits, ids, w, counts, offsets, perm, inv_perm, plan, h, rows, total;
};
FwdLayout fwd_layout(const LayerDims& L, int T, bool pre_norm) {
  FwdLayout f{};
  const size_t a = esz(L.act);
  const size_t N = (size_t)T * L.k, R = N + (size_t)L.S * T;
  size_t o = 0;
  f.xn = o;       o += pre_norm ? al((size_t)T * L.d * a) : 0;
  f.logits = o;   o += al((size_t)T * L.E * 4);
  f.ids = o;      o += al(N * 4);
  f.w = o;        o += al(N * 4);
  f.counts = o;   o += al((size_t)L.E * 4);
  f.offsets = o;  o += al((size_t)(L.E + L.S + 1) * 4);
  f.perm = o;     o += al(N * 4);
  f.inv_perm = o; o += al(N * 4);
  f.plan = o;     o += al(plan_words(T, L.k, L.E, L.S) * 4);
  f.h = o;        o += al(R * L.I * a);
  f.rows = o;     o += al(R * L.d * a);
  f.total = o;
  return f;
}

int32_t check_weights(const LayerDims& L, const moe_expert_weights_t* w) {
  if (!w) return fail(MOE_ERR_INVALID, "weights is NULL");
  REQUIRE_PTR(w->w_gate);
  REQUIRE_PTR(w->w_up);
  REQUIRE_PTR(w->w_down);
  if (L.wdt == MOE_I8) {
    REQUIRE_PTR(w->s_gate);
    REQUIRE_PTR(w->s_up);
    REQUIRE_PTR(w->s_down);
  }
  return MOE_OK;
}

}  // namespace

TimerEvents take_timer(int kernel) {
  TimerEvents ev;
  if (kernel >= 0 && kernel < MOE_KERNEL_COUNT && g_timer_start[kernel]) {
    ev.start = (hipEvent_t)g_timer_start[kernel];
    ev.stop = (hipEvent_t)g_timer_stop[kernel];
    g_timer_start[kernel] = g_timer_stop[kernel] = nullptr;
  }
  return ev;
}

LaunchTimer::LaunchTimer(int kernel, hipStream_t s) : stop_(nullptr), s_(s) {
  const TimerEvents ev = take_timer(kernel);
  if (ev.start) {
    (void)hipEventRecord(ev.start, s);
    stop_ = ev.stop;
  }
}
LaunchTimer::~LaunchTimer() {
  if (stop_) (void)hipEventRecord(stop_, s_);
}

constexpr int kGemvMaxTokens = 8;           // with shared experts
constexpr int kGemvMaxTokensRouted = 32;    // routed experts only, bf16 weights
constexpr int kGemvMaxTokensRoutedI8 = 16;  // routed experts only, int8 weights

int ffn_tile_m(const LayerDims& L, int T) {
  if (L.act == MOE_F32) return 0;
  // The GEMV streams each group's weights once and does its rows in passes of a few rows.
  // A shared expert holds all T rows, so past 8 tokens it needs several passes and the
  // matrix-core GEMM is as fast or faster (DeepSeek shapes: equal layer time at T = 9 and
  // 12, 15% faster at 16).  With routed experts only, groups stay small: on the OLMoE shapes
  // the GEMV is faster up to 32 tokens with bf16 weights (-8% at T = 24, -3% at 32, +9% at
  // 48) and up to 16 with int8 weights (the GEMM is 3% faster at 32).
  const int gemv_max = L.S > 0 ? kGemvMaxTokens
                               : (L.wdt == MOE_I8 ? kGemvMaxTokensRoutedI8 : kGemvMaxTokensRouted);
  return T > gemv_max ? gemm_tile_m(L) : 0;
}

// Just past the GEMV's range with shared experts, the down projection (K = I, the shared
// experts' T rows in a few passes of 4) still streams faster on the GEMV while gate/up is
// faster on the GEMM: DeepSeek shapes, bf16, down 27.9 / 29.4 us on the GEMV against 33.9 /
// 35.7 us on the GEMM at T = 9 / 12, gate/up 51.6 / 55.7 against 47.0 / 51.6 us; at T = 16 and
// with int8 weights the two tie.  The launch plan serves both (the GEMV ignores its tiles).
constexpr int kGemvDownMaxTokensShared = 12;

hipError_t launch_grouped_ffn(const LayerDims& L, int T, const FfnArgs& a, hipStream_t s) {
  if (!ffn_tile_m(L, T)) return launch_gemv_ffn(L, T, a, s);
  if (L.S > 0 && L.wdt == MOE_BF16 && T <= kGemvDownMaxTokensShared) {
    hipError_t e = launch_gemm_ffn(L, T, a, s, kFfnGateUp);
    return e != hipSuccess ? e : launch_gemv_ffn(L, T, a, s, kFfnDown);
  }
  return launch_gemm_ffn(L, T, a, s);
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_version(void) { return 100; }

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_time_next_launch(int32_t kernel, void* start_event, void* stop_event) {
  if (kernel < 0 || kernel >= MOE_KERNEL_COUNT) return fail(MOE_ERR_INVALID, "unknown kernel %d", kernel);
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(MOE_ERR_INVALID, "start_event and stop_event must both be set or both be NULL");
  g_timer_start[kernel] = start_event;
  g_timer_stop[kernel] = stop_event;
  return ok();
}

size_t moe_workspace_bytes(const moe_layer_desc_t* desc, int32_t max_tokens, int32_t which) {
  LayerDims L;
  if (check_desc(desc, &L) != MOE_OK || max_tokens < 0 || check_tokens(L, max_tokens) != MOE_OK)
    return 0;
  const int T = max_tokens;
  const size_t R = (size_t)T * L.k + (size_t)L.S * T;
  switch (which) {
    case MOE_WS_PERMUTE: return al(plan_words(T, L.k, L.E, L.S) * 4);
    case MOE_WS_GROUPED_FFN: return al(R * L.I * esz(L.act));
    case MOE_WS_FORWARD: return fwd_layout(L, T, desc->pre_norm != 0).total;
    default: fail(MOE_ERR_INVALID, "unknown workspace kind %d", which); return 0;
  }
}

int32_t moe_route(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                  const float* router_bias, const float* logits_in, float* logits_out,
                  int32_t* topk_ids, float* topk_w, void* stream) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_w);
  CHECK_ALIGN(logits_out);
  if (!logits_in) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(w_router);
    REQUIRE_PTR(logits_out);
    CHECK_ALIGN(router_bias);
  } else {
    CHECK_ALIGN(logits_in);
  }
  if (T == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const float* lg = logits_in;
  if (!logits_in) {
    if ((e = launch_router_logits(L, T, x, w_router, router_bias, logits_out, s)) != hipSuccess)
      return device_fail(e, "router logits launch");
    lg = logits_out;
  } else if (logits_out && logits_out != logits_in) {
    if ((e = hipMemcpyAsync(logits_out, logits_in, (size_t)T * L.E * 4, hipMemcpyDeviceToDevice, s)) !=
        hipSuccess)
      return device_fail(e, "logits copy");
  }
  if ((e = launch_topk(L, T, lg, topk_ids, topk_w, s)) != hipSuccess) return device_fail(e, "top-k launch");
  return ok();
}

int32_t moe_permute(const moe_layer_desc_t* desc, int32_t T, const int32_t* topk_ids, int32_t* counts,
                    int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* plan, size_t plan_bytes,
                    void* stream) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(perm);
  REQUIRE_PTR(inv_perm);
  REQUIRE_PTR(plan);
  const size_t need = moe_workspace_bytes(desc, T, MOE_WS_PERMUTE);
  if (plan_bytes < need) return fail(MOE_ERR_WORKSPACE, "plan_bytes %zu < %zu", plan_bytes, need);
  if (T == 0) return ok();
  hipError_t e = launch_permute(L, T, topk_ids, counts, offsets, perm, inv_perm, (int32_t*)plan,
                                ffn_tile_m(L, T), (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "permute launch");
  return ok();
}

int32_t moe_grouped_ffn(const moe_layer_desc_t* desc, int32_t T, const void* x,
                        const moe_expert_weights_t* weights, const int32_t* offsets, const int32_t* perm,
                        const void* plan, void* rows, void* ws, size_t ws_bytes, void* stream) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  if ((st = check_weights(L, weights))) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(perm);
  REQUIRE_PTR(plan);
  REQUIRE_PTR(rows);
  REQUIRE_PTR(ws);
  const size_t need = moe_workspace_bytes(desc, T, MOE_WS_GROUPED_FFN);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "ws_bytes %zu < %zu", ws_bytes, need);
  if (T == 0) return ok();
  FfnArgs a{x, weights->w_gate, weights->w_up, weights->w_down, weights->s_gate, weights->s_up,
            weights->s_down, offsets, perm, (const int32_t*)plan, ws, rows};
  if (L.wdt != MOE_I8) a.s_gate = a.s_up = a.s_down = nullptr;
  hipError_t e = launch_grouped_ffn(L, T, a, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "grouped FFN launch");
  return ok();
}

int32_t moe_combine(const moe_layer_desc_t* desc, int32_t T, const void* rows, const int32_t* inv_perm,
                    const float* topk_w, const void* residual, void* y, void* stream) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  REQUIRE_PTR(rows);
  REQUIRE_PTR(inv_perm);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(y);
  CHECK_ALIGN(residual);
  if (T == 0) return ok();
  hipError_t e = launch_combine(L, T, rows, inv_perm, topk_w, residual, y, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "combine launch");
  return ok();
}

int32_t moe_forward(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                    const float* router_bias, const moe_expert_weights_t* weights, const void* residual,
                    void* y, int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                    void* stream) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  if ((st = check_weights(L, weights))) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(y);
  REQUIRE_PTR(ws);
  CHECK_ALIGN(router_bias);
  CHECK_ALIGN(residual);
  CHECK_ALIGN(topk_ids_out);
  CHECK_ALIGN(topk_w_out);
  const size_t need = moe_workspace_bytes(desc, T, MOE_WS_FORWARD);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "ws_bytes %zu < %zu", ws_bytes, need);
  if (T == 0) return ok();

  hipStream_t s = (hipStream_t)stream;
  const FwdLayout f = fwd_layout(L, T, desc->pre_norm != 0);
  char* base = (char*)ws;
  const void* xin = x;
  hipError_t e;
  if (desc->pre_norm) {
    if ((e = launch_rmsnorm(L, T, x, base + f.xn, desc->norm_eps, s)) != hipSuccess)
      return device_fail(e, "rmsnorm launch");
    xin = base + f.xn;
  }
  float* logits = (float*)(base + f.logits);
  int32_t* ids = (int32_t*)(base + f.ids);
  float* w = (float*)(base + f.w);
  int32_t* counts = (int32_t*)(base + f.counts);
  int32_t* offsets = (int32_t*)(base + f.offsets);
  int32_t* perm = (int32_t*)(base + f.perm);
  int32_t* inv_perm = (int32_t*)(base + f.inv_perm);
  int32_t* plan = (int32_t*)(base + f.plan);
  if ((e = launch_router_logits(L, T, xin, w_router, router_bias, logits, s)) != hipSuccess)
    return device_fail(e, "router logits launch");
  if (topk_permute_fusable(L, T)) {
    if ((e = launch_topk_permute(L, T, logits, ids, w, counts, offsets, perm, inv_perm, plan,
                                 ffn_tile_m(L, T), s)) != hipSuccess)
      return device_fail(e, "top-k + permute launch");
  } else {
    if ((e = launch_topk(L, T, logits, ids, w, s)) != hipSuccess) return device_fail(e, "top-k launch");
    if ((e = launch_permute(L, T, ids, counts, offsets, perm, inv_perm, plan, ffn_tile_m(L, T), s)) !=
        hipSuccess)
      return device_fail(e, "permute launch");
  }
  FfnArgs a{xin, weights->w_gate, weights->w_up, weights->w_down, weights->s_gate, weights->s_up,
            weights->s_down, offsets, perm, plan, base + f.h, base + f.rows};
  if (L.wdt != MOE_I8) a.s_gate = a.s_up = a.s_down = nullptr;
  if ((e = launch_grouped_ffn(L, T, a, s)) != hipSuccess) return device_fail(e, "grouped FFN launch");
  if ((e = launch_combine(L, T, base + f.rows, inv_perm, w, residual, y, s)) != hipSuccess)
    return device_fail(e, "combine launch");
  if (topk_ids_out &&
      (e = hipMemcpyAsync(topk_ids_out, ids, (size_t)T * L.k * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return device_fail(e, "topk_ids copy");
  if (topk_w_out &&
      (e = hipMemcpyAsync(topk_w_out, w, (size_t)T * L.k * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return device_fail(e, "topk_w copy");
  return ok();
}

}  // extern "C"
