// The exported C ABI of libmoe (declared in include/moe.h): argument checks, workspace
// layout, and the choice between the decode (grouped GEMV) and prefill (MFMA grouped GEMM)
// kernels.  Every check runs on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
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

// Which kernel family serves a layer's two FFN launches at T tokens.  Three regimes, by the
// rows a group holds (a routed expert T*k/E on average, a shared expert all T):
//  * the VALU GEMV while groups hold a few rows: its dot products cost less than the matrix
//    cores' 16-token tiles (OLMoE shapes: gate/up at T=8 66.5 against 69.3 us on the
//    matrix-core GEMV, int8 36 against 42 us);
//  * the matrix-core GEMV (same weight streaming, MFMA math, rows in chunks of 16) while the
//    groups stay within a chunk or two: OLMoE layer -4% at T=32, -13% at T=48, -11% at T=64
//    against the GEMM, +2% at T=128 (mean 16 rows); int8 -7% at T=24, -2% at 48, +1% at 64.  With
//    shared experts (DeepSeek shapes) from T=8 (-4% against the VALU GEMV) to T=16 (-7%
//    against the GEMM; -9 to -10% at T=9 and 12; +3% at T=32, where a shared expert's 32
//    rows take two chunks); int8 -7% at T=8 and 16;
//  * the LDS-ring GEMM beyond.
// The matrix-core GEMV needs bf16 activations and d, I multiples of 64; other layers keep
// the VALU GEMV up to 8 tokens with shared experts, 32 (bf16 weights) or 16 (int8) without.
enum class FfnPath { kGemv, kGemvMfma, kGemm };

constexpr int kGemvMaxTokensShared = 7;     // VALU GEMV with shared experts
constexpr int kGemvRowsRouted = 3;          // VALU GEMV without: mean rows per routed group,
constexpr int kGemvRowsRoutedI8 = 2;        //   bf16 / int8 weights
constexpr int kMfmaMaxTokensShared = 16;    // matrix-core GEMV with shared experts
constexpr int kMfmaRowsRouted = 8;          // matrix-core GEMV without: mean rows per group
constexpr int kMfmaRowsRoutedI8 = 6;
constexpr int kGemvMaxTokensNoMfma[2] = {32, 16};  // layers the matrix-core GEMV cannot take:
constexpr int kGemvMaxTokensNoMfmaShared = 8;      //   VALU GEMV limits (bf16, int8 weights)

FfnPath ffn_path(const LayerDims& L, int T) {
  if (L.act == MOE_F32) return FfnPath::kGemv;
  const bool i8 = L.wdt == MOE_I8;
  const long tk = (long)T * L.k, E = L.E;
  if (L.d % 64 != 0 || L.I % 64 != 0) {
    const int gemv_max = L.S > 0 ? kGemvMaxTokensNoMfmaShared : kGemvMaxTokensNoMfma[i8];
    return T > gemv_max ? FfnPath::kGemm : FfnPath::kGemv;
  }
  if (L.S > 0) {
    if (T <= kGemvMaxTokensShared) return FfnPath::kGemv;
    return T <= kMfmaMaxTokensShared ? FfnPath::kGemvMfma : FfnPath::kGemm;
  }
  if (tk <= (i8 ? kGemvRowsRoutedI8 : kGemvRowsRouted) * E) return FfnPath::kGemv;
  return tk <= (i8 ? kMfmaRowsRoutedI8 : kMfmaRowsRouted) * E ? FfnPath::kGemvMfma : FfnPath::kGemm;
}

// The launch plan carries M-tiles only for the GEMM; both GEMVs read its group list alone.
int ffn_tile_m(const LayerDims& L, int T) {
  return ffn_path(L, T) == FfnPath::kGemm ? gemm_tile_m(L) : 0;
}

hipError_t launch_grouped_ffn(const LayerDims& L, int T, const FfnArgs& a, hipStream_t s) {
  switch (ffn_path(L, T)) {
    case FfnPath::kGemv: return launch_gemv_ffn(L, T, a, s);
    case FfnPath::kGemvMfma: return launch_gemv_mfma_ffn(L, T, a, s);
    default: return launch_gemm_ffn(L, T, a, s);
  }
}

// ---------------------------------------------------------------------------------------
// Scratch memory of moe_forward_noalloc, for callers that cannot allocate.  One copy per GPU:
// the array is part of the library's device code object, so each device the library runs on
// holds its own copy from the code object's load until the process ends.  In host code the
// array's name is only a host-side stand-in; its device address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is ever handed to kernels.  Every call on a device shares the device's copy, which
// keeps the last call's contents; nothing in it has to start at zero (each kernel writes
// what a later one reads).
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)128 << 20;  // 128 MiB: the OLMoE-shaped layer up
                                                      // to about 2,700 tokens
__attribute__((used)) static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device ordinal

// The device `stream` belongs to, and that device's address of `scratch` (looked up on the
// first call for the device, with the device made current for the lookup).
int32_t scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return device_fail(e, "hipStreamGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device ordinal %d beyond the %d this library tracks", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return device_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return device_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return device_fail(e2, "hipSetDevice");
    }
    if (e != hipSuccess) return device_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u)) return fail(MOE_ERR_DEVICE, "scratch address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

int32_t forward_impl(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                     const float* router_bias, const moe_expert_weights_t* weights,
                     const void* residual, void* y, int32_t* topk_ids_out, float* topk_w_out,
                     void* ws, size_t ws_bytes, void* stream, bool use_scratch);

}  // namespace

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

int32_t moe_ffn_kernel(const moe_layer_desc_t* desc, int32_t T) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st != MOE_OK) return st;
  if (T < 1) return fail(MOE_ERR_INVALID, "T = %d: the kernel choice needs at least one token", T);
  if ((st = check_tokens(L, T)) != MOE_OK) return st;
  switch (ffn_path(L, T)) {
    case FfnPath::kGemv: return MOE_FFN_GEMV;
    case FfnPath::kGemvMfma: return MOE_FFN_GEMV_MFMA;
    default: return MOE_FFN_GEMM;
  }
}

int32_t moe_route(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                  const float* router_bias, const float* logits_in, float* logits_out,
                  int32_t* topk_ids, float* topk_w, void* stream) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  if (desc->pre_norm)
    return fail(MOE_ERR_UNSUPPORTED,
                "pre_norm = 1: moe_route takes x (or logits_in) as given; only moe_forward applies "
                "the RMSNorm, so pass the normalised input with pre_norm = 0");
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
  if (desc->pre_norm)
    return fail(MOE_ERR_UNSUPPORTED,
                "pre_norm = 1: moe_grouped_ffn takes x as given; only moe_forward applies the "
                "RMSNorm, so pass the normalised input with pre_norm = 0");
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
  return forward_impl(desc, T, x, w_router, router_bias, weights, residual, y, topk_ids_out, topk_w_out,
                      ws, ws_bytes, stream, /*use_scratch=*/false);
}

int32_t moe_forward_noalloc(const moe_layer_desc_t* desc, int32_t T, const void* x,
                            const void* w_router, const float* router_bias,
                            const moe_expert_weights_t* weights, const void* residual, void* y,
                            int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  return forward_impl(desc, T, x, w_router, router_bias, weights, residual, y, topk_ids_out, topk_w_out,
                      nullptr, 0, stream, /*use_scratch=*/true);
}

}  // extern "C"

namespace moe {
namespace {

int32_t forward_impl(const moe_layer_desc_t* desc, int32_t T, const void* x, const void* w_router,
                     const float* router_bias, const moe_expert_weights_t* weights,
                     const void* residual, void* y, int32_t* topk_ids_out, float* topk_w_out,
                     void* ws, size_t ws_bytes, void* stream, bool use_scratch) {
  LayerDims L;
  int32_t st = check_desc(desc, &L);
  if (st) return st;
  if ((st = check_tokens(L, T))) return st;
  if ((st = check_weights(L, weights))) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(y);
  if (!use_scratch) REQUIRE_PTR(ws);
  CHECK_ALIGN(router_bias);
  CHECK_ALIGN(residual);
  CHECK_ALIGN(topk_ids_out);
  CHECK_ALIGN(topk_w_out);
  const size_t need = moe_workspace_bytes(desc, T, MOE_WS_FORWARD);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(MOE_ERR_WORKSPACE,
                  "T = %d needs %zu bytes of workspace; the library's static scratch holds %zu "
                  "(use moe_forward with a caller workspace)",
                  T, need, kScratchBytes);
    if (T == 0) return ok();
    if ((st = scratch_for_stream((hipStream_t)stream, &ws))) return st;
    ws_bytes = kScratchBytes;
  }
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
  if (ffn_path(L, T) == FfnPath::kGemv && gemv_down_combine_fits(L, T)) {
    // decode sizes: the down projection and the combine in one launch
    if ((e = launch_gemv_ffn_combine(L, T, a, inv_perm, w, residual, y, s)) != hipSuccess)
      return device_fail(e, "grouped FFN + combine launch");
  } else {
    if ((e = launch_grouped_ffn(L, T, a, s)) != hipSuccess) return device_fail(e, "grouped FFN launch");
    if ((e = launch_combine(L, T, base + f.rows, inv_perm, w, residual, y, s)) != hipSuccess)
      return device_fail(e, "combine launch");
  }
  if (topk_ids_out &&
      (e = hipMemcpyAsync(topk_ids_out, ids, (size_t)T * L.k * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return device_fail(e, "topk_ids copy");
  if (topk_w_out &&
      (e = hipMemcpyAsync(topk_w_out, w, (size_t)T * L.k * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return device_fail(e, "topk_w copy");
  return ok();
}

}  // namespace
}  // namespace moe
