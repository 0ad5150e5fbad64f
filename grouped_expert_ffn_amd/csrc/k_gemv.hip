// Grouped GEMV for decode sizes: every touched expert in one launch, weights streamed once.
//
// At decode sizes an expert sees one to a few rows, so the layer is bound by reading the
// touched experts' weights from HBM (the switchyard page's decode kernel is "a grouped GEMV"
// that streams expert weights, §02 "One launch for all experts").  The kernel is laid out
// for that: blockIdx.x walks the touched groups of the launch plan, blockIdx.y a block of
// NB output channels.  A group of LPC lanes owns one output channel and reads its weight row
// in LPC*16-byte coalesced runs; the group's rows of activations (gathered through perm for
// gate/up, contiguous h rows for down) sit in LDS and are re-read per weight chunk.  The
// channel's partial sums are reduced across its LPC lanes by xor-shuffles, then the
// epilogue applies the int8 scale, the SwiGLU (gate/up) and rounds to the activation type.
//
// Weight/activation types: f32 x f32 (fp32 FMA), bf16 x bf16 (v_dot2_f32_bf16), int8 x bf16
// (int8 -> bf16 is exact for |q| <= 127, then v_dot2_f32_bf16; the per-channel scale
// multiplies the fp32 sum once).
#include "moe_internal.h"

namespace moe {

namespace {

struct GemvArgs {
  const void* in;   // gate/up: x [T, K] gathered by token; down: h [R, K] by row
  const void* w0;   // [G, N, K]
  const void* w1;   // up weights for gate/up, else unused
  const float* s0;  // int8 scales [G, N]
  const float* s1;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* plan;
  void* out;        // [R, N]
  int K, N, k, E, kc;  // kc: K columns staged in LDS at a time
};

constexpr int kLPC = 8;  // lanes per output channel
constexpr int kMB = 8;   // rows per pass (<= kLPC)

template <typename WT> struct WTraits;
template <> struct WTraits<float> { static constexpr int V = 4; };     // per 16-byte load
template <> struct WTraits<uint16_t> { static constexpr int V = 8; };
template <> struct WTraits<int8_t> { static constexpr int V = 16; };

// 16 int8 weights -> 8 packed bf16 pairs (exact)
__device__ __forceinline__ void i8x16_to_bf16(const uint4& q, uint32_t (&o)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t v = (int32_t)w[i];
    const float b0 = (float)((v << 24) >> 24), b1 = (float)((v << 16) >> 24);
    const float b2 = (float)((v << 8) >> 24), b3 = (float)(v >> 24);
    o[2 * i] = pack_bf16x2(b0, b1);
    o[2 * i + 1] = pack_bf16x2(b2, b3);
  }
}

// acc += <weight chunk, activation chunk> for one row; xs points at the row's chunk in LDS
template <typename AT, typename WT> struct Dot;
template <> struct Dot<float, float> {
  typedef uint4 W;
  __device__ static W prep(const uint4& q) { return q; }
  __device__ static float run(const W& w, const unsigned char* xs, float acc) {
    const float4 x = *reinterpret_cast<const float4*>(xs);
    acc = fmaf(__uint_as_float(w.x), x.x, acc);
    acc = fmaf(__uint_as_float(w.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.z), x.z, acc);
    acc = fmaf(__uint_as_float(w.w), x.w, acc);
    return acc;
  }
};
template <> struct Dot<uint16_t, uint16_t> {
  typedef uint4 W;
  __device__ static W prep(const uint4& q) { return q; }
  __device__ static float run(const W& w, const unsigned char* xs, float acc) {
    const uint4 x = *reinterpret_cast<const uint4*>(xs);
    acc = dot2_bf16(w.x, x.x, acc);
    acc = dot2_bf16(w.y, x.y, acc);
    acc = dot2_bf16(w.z, x.z, acc);
    acc = dot2_bf16(w.w, x.w, acc);
    return acc;
  }
};
template <> struct Dot<uint16_t, int8_t> {
  struct W {
    uint32_t v[8];
  };
  __device__ static W prep(const uint4& q) {
    W w;
    i8x16_to_bf16(q, w.v);
    return w;
  }
  __device__ static float run(const W& w, const unsigned char* xs, float acc) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(xs);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xs + 16);
    acc = dot2_bf16(w.v[0], x0.x, acc);
    acc = dot2_bf16(w.v[1], x0.y, acc);
    acc = dot2_bf16(w.v[2], x0.z, acc);
    acc = dot2_bf16(w.v[3], x0.w, acc);
    acc = dot2_bf16(w.v[4], x1.x, acc);
    acc = dot2_bf16(w.v[5], x1.y, acc);
    acc = dot2_bf16(w.v[6], x1.z, acc);
    acc = dot2_bf16(w.v[7], x1.w, acc);
    return acc;
  }
};

// MODE 0: h = silu(W0 x) * (W1 x);  MODE 1: out = W0 h
// grid: (slots, ceil(N / NB)); block 256; dynamic LDS kMB * kc * sizeof(AT)
template <int MODE, typename AT, typename WT>
__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a) {
  constexpr int CPW = kWave / kLPC;  // channels per wavefront
  constexpr int NB = 4 * CPW;        // channels per block
  constexpr int V = WTraits<WT>::V;  // elements per lane step
  constexpr int XB = V * (int)sizeof(AT);  // activation bytes per lane step
  typedef Dot<AT, WT> D;
  extern __shared__ __align__(16) unsigned char xs[];

  const int slot = blockIdx.x;
  if (slot >= a.plan[0]) return;
  const int g = a.plan[kPlanHeader + slot];
  const int r0 = a.offsets[g];
  const int M = a.offsets[g + 1] - r0;
  const int K = a.K, N = a.N;

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int q = lane % kLPC, ci = lane / kLPC;
  const int n = blockIdx.y * NB + wave * CPW + ci;
  const bool nvalid = n < N;
  const size_t wrow = ((size_t)g * N + (nvalid ? n : N - 1)) * K;
  const WT* w0 = reinterpret_cast<const WT*>(a.w0) + wrow;
  const WT* w1 = MODE == 0 ? reinterpret_cast<const WT*>(a.w1) + wrow : nullptr;
  const AT* in = reinterpret_cast<const AT*>(a.in);
  const int row_bytes = a.kc * (int)sizeof(AT);

  for (int m0 = 0; m0 < M; m0 += kMB) {
    const int mb = min(kMB, M - m0);
    float acc0[kMB], acc1[kMB];
#pragma unroll
    for (int m = 0; m < kMB; ++m) acc0[m] = acc1[m] = 0.f;

    for (int k0 = 0; k0 < K; k0 += a.kc) {
      const int kc = min(a.kc, K - k0);
      // stage rows m0 .. m0+mb-1, columns k0 .. k0+kc-1 of the input into LDS
      __syncthreads();
      const int chunks = kc * (int)sizeof(AT) / 16;
      for (int i = threadIdx.x; i < mb * chunks; i += blockDim.x) {
        const int m = i / chunks, c = i % chunks;
        const int r = r0 + m0 + m;
        size_t src_row;
        if (MODE == 0)
          src_row = (g < a.E) ? (size_t)(a.perm[r] / a.k) : (size_t)(r - r0);
        else
          src_row = (size_t)r;
        const uint4* src = reinterpret_cast<const uint4*>(in + src_row * K + k0);
        reinterpret_cast<uint4*>(xs + m * row_bytes)[c] = src[c];
      }
      __syncthreads();

#pragma unroll 4
      for (int c = q * V; c < kc; c += kLPC * V) {
        const typename D::W wa = D::prep(*reinterpret_cast<const uint4*>(w0 + k0 + c));
        typename D::W wb;
        if (MODE == 0) wb = D::prep(*reinterpret_cast<const uint4*>(w1 + k0 + c));
        const unsigned char* xp = xs + c * (int)sizeof(AT);
#pragma unroll
        for (int m = 0; m < kMB; ++m) {
          if (m < mb) {
            acc0[m] = D::run(wa, xp + m * row_bytes, acc0[m]);
            if (MODE == 0) acc1[m] = D::run(wb, xp + m * row_bytes, acc1[m]);
          }
        }
      }
      (void)XB;
    }
    // reduce over the channel's lanes
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
#pragma unroll
      for (int off = kLPC / 2; off >= 1; off >>= 1) {
        acc0[m] += __shfl_xor(acc0[m], off, kWave);
        if (MODE == 0) acc1[m] += __shfl_xor(acc1[m], off, kWave);
      }
    }
    // lane q of the channel's group writes row m0 + q
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
      if (nvalid && m < mb && q == m) {
        float v0 = acc0[m];
        const size_t o = (size_t)(r0 + m0 + m) * N + n;
        if (MODE == 0) {
          float v1 = acc1[m];
          if (a.s0) {
            v0 *= a.s0[(size_t)g * N + n];
            v1 *= a.s1[(size_t)g * N + n];
          }
          Act<AT>::store(reinterpret_cast<AT*>(a.out), o, silu(v0) * v1);
        } else {
          if (a.s0) v0 *= a.s0[(size_t)g * N + n];
          Act<AT>::store(reinterpret_cast<AT*>(a.out), o, v0);
        }
      }
    }
  }
}

template <int MODE, typename AT, typename WT>
hipError_t run_gemv(const GemvArgs& a, int slots, hipStream_t s) {
  constexpr int NB = 4 * (kWave / kLPC);
  dim3 grid(slots, (a.N + NB - 1) / NB);
  const size_t lds = (size_t)kMB * a.kc * sizeof(AT);
  LaunchTimer timer(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, s);
  k_gemv<MODE, AT, WT><<<grid, 256, lds, s>>>(a);
  return hipGetLastError();
}

// K columns staged per pass: a multiple of the lane-group span that keeps LDS <= 32 KiB
int stage_cols(int K, int esz, int span) {
  int kc = (32 * 1024) / (kMB * esz);
  kc = (kc / span) * span;
  return kc >= K ? K : kc;
}

}  // namespace

hipError_t launch_gemv_ffn(const LayerDims& L, int T, const FfnArgs& f, hipStream_t s) {
  const int slots = (T * L.k < L.E ? T * L.k : L.E) + L.S;
  GemvArgs a{};
  a.offsets = f.offsets;
  a.perm = f.perm;
  a.plan = f.plan;
  a.k = L.k;
  a.E = L.E;
  hipError_t err;
  const int esz = L.act == MOE_F32 ? 4 : 2;
  const int span = kLPC * (L.wdt == MOE_I8 ? 16 : (L.wdt == MOE_F32 ? 4 : 8));

  // gate/up + SwiGLU
  a.in = f.x;
  a.w0 = f.w_gate;
  a.w1 = f.w_up;
  a.s0 = f.s_gate;
  a.s1 = f.s_up;
  a.out = f.h;
  a.K = L.d;
  a.N = L.I;
  a.kc = stage_cols(L.d, esz, span);
  if (L.act == MOE_F32)
    err = run_gemv<0, float, float>(a, slots, s);
  else if (L.wdt == MOE_I8)
    err = run_gemv<0, uint16_t, int8_t>(a, slots, s);
  else
    err = run_gemv<0, uint16_t, uint16_t>(a, slots, s);
  if (err != hipSuccess) return err;

  // down
  a.in = f.h;
  a.w0 = f.w_down;
  a.w1 = nullptr;
  a.s0 = f.s_down;
  a.s1 = nullptr;
  a.out = f.rows;
  a.K = L.I;
  a.N = L.d;
  a.kc = stage_cols(L.I, esz, span);
  if (L.act == MOE_F32)
    err = run_gemv<1, float, float>(a, slots, s);
  else if (L.wdt == MOE_I8)
    err = run_gemv<1, uint16_t, int8_t>(a, slots, s);
  else
    err = run_gemv<1, uint16_t, uint16_t>(a, slots, s);
  return err;
}

}  // namespace moe
