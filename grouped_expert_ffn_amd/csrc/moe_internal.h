// Internal declarations of libmoe: device helpers and kernel launchers.
// Everything here is gfx950 (CDNA4, wave64) code; nothing is exported.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// -------------------------------------------------------------------------------------
// scalar conversions
// -------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
// two floats -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 += a.lo*b.lo + a.hi*b.hi over packed bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// 8 int8 weights -> 8 bf16 (exact for |q| <= 127)
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(const uint2& q) {
  uint32_t o[4];
  const uint32_t w[2] = {q.x, q.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int32_t v = (int32_t)w[i];
    o[2 * i] = pack_bf16x2((float)((v << 24) >> 24), (float)((v << 16) >> 24));
    o[2 * i + 1] = pack_bf16x2((float)((v << 8) >> 24), (float)(v >> 24));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Activation element access for the two activation types.
template <typename AT> struct Act;
template <> struct Act<float> {
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static void store(float* p, size_t i, float v) { p[i] = v; }
  __device__ static float round(float v) { return v; }  // the value a store then load gives
};
template <> struct Act<uint16_t> {
  __device__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  __device__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// -------------------------------------------------------------------------------------
// wave-level helpers
// -------------------------------------------------------------------------------------
// DPP lane moves (VALU modifiers, no LDS round trip).  Controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror (lane i <-> 7-i within 8) = 0x141,
// row_mirror (lane i <-> 15-i within 16) = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
// Sum over each aligned group of 8 lanes; every lane of the group gets the same bits
// (each step adds a value and its partner, and fp addition is commutative).
// A dot-product sum about to be read by DPP lane moves.  On gfx950 a DPP read two
// instructions after v_dot2c_f32_bf16 wrote its source register has returned the value from
// before that write (a row sum came out missing its last term), and the compiler may space the
// two by only two instructions.  The asm ties the value, so nothing is scheduled across it, and
// adds three wait states.
__device__ __forceinline__ float settle_dot(float v) {
  asm volatile("s_nop 2" : "+v"(v));
  return v;
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<0x140>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}
__device__ __forceinline__ float readlane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Wave-wide sum / max, identical (wave-uniform) in every lane, fixed order.
__device__ __forceinline__ float wave_sum_u(float v) {
  v = sum16(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}
__device__ __forceinline__ float wave_max_u(float v) {
  v = max16(v);
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}
// -------------------------------------------------------------------------------------
// plan buffer written by the permute kernel (int32 words)
// -------------------------------------------------------------------------------------
//   [0] number of groups with rows (touched routed experts + shared experts)
//   [1] number of M-tiles in the tile list
//   [2] M-tile height the tile list was built for
//   [3] capacity C: routed group g holds min(rows, C) rows (0 = no limit)
//   [4 .. 4+E+S)            touched group ids, ascending (routed first, then shared)
//   [4+E+S .. + 2*max_tiles) tile list: (group, first row within the group)
//   then, for the multi-workgroup sort, one expert histogram per chunk of kPermChunk rows
//   (turned in place into each chunk's per-expert base by a scan), then the E expert totals
constexpr int kPlanHeader = 4;
constexpr int kMinTileM = 16;
constexpr int kPermChunk = 1024;  // rows per workgroup of the multi-workgroup sort
constexpr int kSmallSortRows = kWave;  // rows (T*k) the one-wavefront sort takes
inline size_t plan_max_tiles(int T, int k, int E, int S) {
  const size_t N = (size_t)T * k;
  return N / kMinTileM + (size_t)E + (size_t)S * ((T + kMinTileM - 1) / kMinTileM) + 1;
}
inline size_t plan_hist_offset(int T, int k, int E, int S) {
  return kPlanHeader + (size_t)(E + S) + 2 * plan_max_tiles(T, k, E, S);
}
inline size_t plan_words(int T, int k, int E, int S) {
  const size_t chunks = ((size_t)T * k + kPermChunk - 1) / kPermChunk;
  return plan_hist_offset(T, k, E, S) + (chunks + 1) * (size_t)E;
}

// -------------------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// -------------------------------------------------------------------------------------
// Brackets one kernel launch with the caller's events when moe_time_next_launch armed it.
// Timing hook (moe_time_next_launch).  A step that is one launch goes through launch(): the
// armed events are handed to the launch itself (hipExtLaunchKernelGGL records them from the
// dispatch, i.e. the kernel's own start and end).  A step of several launches is bracketed
// by a LaunchTimer, which records the events on the stream around them.
struct TimerEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
TimerEvents take_timer(int kernel);  // the events armed for `kernel` (then disarmed), or nulls

template <typename F, typename... Args>
hipError_t launch(int kernel, F f, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
  const TimerEvents ev = take_timer(kernel);
  hipExtLaunchKernelGGL(f, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
  return hipGetLastError();
}

// Raise a kernel's dynamic-LDS limit once per device (the attribute belongs to the current
// device; the flags are indexed by device ordinal and safe to race on).
constexpr int kMaxDevices = 64;
typedef std::atomic<bool> LdsFlags[kMaxDevices];
template <typename F>
hipError_t set_lds(F* kernel, size_t bytes, LdsFlags& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[dev].store(true, std::memory_order_release);
  return e;
}

class LaunchTimer {
 public:
  LaunchTimer(int kernel, hipStream_t s);
  ~LaunchTimer();
 private:
  hipEvent_t stop_;
  hipStream_t s_;
};

struct LayerDims {
  int d, E, k, I, S, renorm, act, wdt;
  float cf;  // capacity factor, 0 = dropless
};

// Rows each routed expert keeps: ceil(cf * T * k / E) formed in double in that order, 0 for
// no limit.  An expert never holds more than T rows (a token picks it at most once), so the
// value is capped at T, which changes nothing.
inline int capacity_rows(const LayerDims& L, int T) {
  if (!(L.cf > 0.f)) return 0;
  const double c = std::ceil((double)L.cf * T * L.k / L.E);
  return c >= (double)T ? T : (int)c;
}

hipError_t launch_rmsnorm(const LayerDims& L, int T, const void* x, void* xn, float eps,
                          hipStream_t s);
hipError_t launch_router_logits(const LayerDims& L, int T, const void* x, const void* w_router,
                                const float* bias, float* logits, hipStream_t s);
hipError_t launch_topk(const LayerDims& L, int T, const float* logits, int32_t* ids, float* w,
                       hipStream_t s);
hipError_t launch_permute(const LayerDims& L, int T, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* plan,
                          int tile_m, hipStream_t s);

// Top-k and the sort fused in one workgroup (small T*k only; see topk_permute_fusable).
bool topk_permute_fusable(const LayerDims& L, int T);
hipError_t launch_topk_permute(const LayerDims& L, int T, const float* logits, int32_t* ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_perm, int32_t* plan, int tile_m, hipStream_t s);

struct FfnArgs {
  const void* x;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* plan;
  void* h;
  void* rows;
};
// M-tile height the grouped FFN will use for T tokens (0: a GEMV path, no tile list needed).
int ffn_tile_m(const LayerDims& L, int T);
hipError_t launch_grouped_ffn(const LayerDims& L, int T, const FfnArgs& a, hipStream_t s);
// the FFN's two launches (gate/up + SwiGLU, then down) on one kernel family: the VALU GEMV,
// the matrix-core GEMV (bf16 activations, d and I multiples of 64), the MFMA GEMM
hipError_t launch_gemv_ffn(const LayerDims& L, int T, const FfnArgs& a, hipStream_t s);
hipError_t launch_gemv_mfma_ffn(const LayerDims& L, int T, const FfnArgs& a, hipStream_t s);
// moe_forward at decode sizes: the VALU GEMV's gate/up, then the down projection and the
// combine as one launch (y bit-identical to launch_gemv_ffn + launch_combine).  Applies when
// the layer is on the VALU GEMV path and gemv_down_combine_fits(L, T).
bool gemv_down_combine_fits(const LayerDims& L, int T);
hipError_t launch_gemv_ffn_combine(const LayerDims& L, int T, const FfnArgs& a, const int32_t* inv_perm,
                                   const float* topk_w, const void* residual, void* y, hipStream_t s);
hipError_t launch_gemm_ffn(const LayerDims& L, int T, const FfnArgs& a, hipStream_t s);
int gemm_tile_m(const LayerDims& L);

hipError_t launch_combine(const LayerDims& L, int T, const void* rows, const int32_t* inv_perm,
                          const float* topk_w, const void* residual, void* y, hipStream_t s);

}  // namespace moe
