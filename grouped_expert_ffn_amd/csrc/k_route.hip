// Router logits, top-k gating and the RMSNorm prologue.
//
// Router: logits[t,e] = sum_c x[t,c] W_r[e,c] + b[e] with fp32 accumulation.  Past 64 tokens,
// bf16 layers whose d is a multiple of 32 use the matrix cores (k_router_mfma below).
// Otherwise a block of four wavefronts stages a few token rows in LDS; each wavefront first
// issues the loads of a whole W_r row (16 bytes per lane per load, all in flight together),
// then reduces with DPP.  Up to 64 tokens every wavefront owns one expert (many small
// blocks, so the router matrix is read by many CUs at once); beyond, a block owns all
// experts for its tokens and prefetches the next expert's row while reducing the current.
//
// Top-k: one wavefront per token (the switchyard page routes each token in one warp, §02
// "Route and sort").  Each lane holds up to four logits; k rounds of wave-wide max / min
// reductions pick the slots, largest first, equal logits going to the lower expert id.  The
// softmax runs over all E logits; sums and the max use DPP trees in a fixed order.
#include "moe_internal.h"
#include "topk.h"

namespace moe {

constexpr int kRouteTB = 8;  // tokens per router block (upper bound)
constexpr int kRouterMfmaMinT = 64;  // the matrix-core router serves T above this

namespace {

template <typename AT>
__device__ __forceinline__ float dot_chunk(const uint4& w, const uint4& x);
template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(const uint4& w, const uint4& x) {
  float a = 0.f;
  a = dot2_bf16(w.x, x.x, a);
  a = dot2_bf16(w.y, x.y, a);
  a = dot2_bf16(w.z, x.z, a);
  a = dot2_bf16(w.w, x.w, a);
  return a;
}
template <>
__device__ __forceinline__ float dot_chunk<float>(const uint4& w, const uint4& x) {
  float a = __uint_as_float(w.x) * __uint_as_float(x.x);
  a = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), a);
  a = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), a);
  a = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), a);
  return a;
}

// grid: (ceil(T / tb_max), ceil(E / (4 * epw))); block 256; dynamic LDS tb_max * d * sizeof(AT)
template <typename AT>
__global__ __launch_bounds__(256) void k_router_logits(int T, int d, int E, int epw, int tb_max,
                                                       const AT* __restrict__ x,
                                                       const AT* __restrict__ w,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ logits) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int R = 8;                // 16-byte chunks per lane kept in flight
  constexpr int V = 16 / sizeof(AT);  // elements per 16-byte chunk
  const int t0 = blockIdx.x * tb_max;
  const int tb = min(tb_max, T - t0);
  const int row_chunks = d / V;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int e0 = (blockIdx.y * 4 + wave) * epw;

  uint4 wv[R];
  auto load_slice = [&](int e, int c0) {
    const uint4* wr = reinterpret_cast<const uint4*>(w + (size_t)min(e, E - 1) * d);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = c0 + lane + kWave * i;
      wv[i] = c < row_chunks ? wr[c] : make_uint4(0, 0, 0, 0);
    }
  };
  load_slice(e0, 0);  // in flight while the activations are staged
  // the first expert's bias, fetched now rather than after the dot products
  float b_next = (bias && e0 < E) ? bias[e0] : 0.f;

  // token rows -> LDS, eight loads per thread in flight before their stores
  uint4* xs = reinterpret_cast<uint4*>(smem);
  const uint4* xg = reinterpret_cast<const uint4*>(x + (size_t)t0 * d);
  const int total = tb * row_chunks;
  for (int i0 = threadIdx.x; i0 < total; i0 += 8 * blockDim.x) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * blockDim.x;
      v[u] = i < total ? xg[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * blockDim.x;
      if (i < total) xs[i] = v[u];
    }
  }
  __syncthreads();

  for (int ei = 0; ei < epw; ++ei) {
    const int e = e0 + ei;
    if (e >= E) break;
    float acc[kRouteTB];
#pragma unroll
    for (int t = 0; t < kRouteTB; ++t) acc[t] = 0.f;
    for (int c0 = 0; c0 < row_chunks; c0 += kWave * R) {
      if (c0 > 0) load_slice(e, c0);
      // A step whose 64 chunks all lie in the row has no per-lane test, so its LDS reads are
      // issued together; token rows past this block's are clamped into the staged rows (their
      // sums are never stored).  Only a partial last step tests each lane.
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int cb = c0 + kWave * i;
        if (cb >= row_chunks) break;
        const int c = cb + lane;
        if (cb + kWave <= row_chunks) {
#pragma unroll
          for (int t = 0; t < kRouteTB; ++t) {
            const int tr = t < tb ? t : tb - 1;
            acc[t] += dot_chunk<AT>(wv[i], xs[tr * row_chunks + c]);
          }
        } else if (c < row_chunks) {
#pragma unroll
          for (int t = 0; t < kRouteTB; ++t) {
            const int tr = t < tb ? t : tb - 1;
            acc[t] += dot_chunk<AT>(wv[i], xs[tr * row_chunks + c]);
          }
        }
      }
    }
    if (ei + 1 < epw && e + 1 < E) load_slice(e + 1, 0);  // next expert's row
    const float b = b_next;
    if (bias && ei + 1 < epw && e + 1 < E) b_next = bias[e + 1];
    // the 8 token sums over the wavefront, halving the values each lane carries: lanes
    // exchange half of them at strides 32, 16 and 8 (then lane l carries token (l >> 3) & 7),
    // and the remaining single value is summed at strides 4, 2 and 1 (fixed order)
    static_assert(kRouteTB == 8, "butterfly over 8 token sums");
    const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
    float v4[4], v2[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float mine = h5 ? acc[j + 4] : acc[j], give = h5 ? acc[j] : acc[j + 4];
      v4[j] = mine + __uint_as_float(xor_lane<32>(__float_as_uint(give)));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float mine = h4 ? v4[j + 2] : v4[j], give = h4 ? v4[j] : v4[j + 2];
      v2[j] = mine + __uint_as_float(xor_lane<16>(__float_as_uint(give)));
    }
    float tot = (h3 ? v2[1] : v2[0]) + __uint_as_float(xor_lane<8>(__float_as_uint(h3 ? v2[0] : v2[1])));
    tot += __uint_as_float(xor_lane<4>(__float_as_uint(tot)));
    tot += __uint_as_float(xor_lane<2>(__float_as_uint(tot)));
    tot += __uint_as_float(xor_lane<1>(__float_as_uint(tot)));
    const int t = lane >> 3;
    if ((lane & 7) == 0 && t < tb) logits[(size_t)(t0 + t) * E + e] = tot + b;
  }
}

// Router logits on the matrix cores, for bf16 layers past decode sizes (d a multiple of 32).
// A block owns 16 tokens and 16*NJ experts (blockIdx.y); its 8 wavefronts split K into 8
// contiguous slices and each accumulates the 16 x 16*NJ partial logits of its slice with
// v_mfma_f32_16x16x32_bf16, reading both operands straight from global memory (token rows
// and router rows from L2).  The eight partials are summed in LDS in a fixed order.
// grid: (ceil(T / 16), ceil(E / (16 * NJ))); block 512
constexpr int kRouterMfmaWaves = 8;
template <int NJ>
__global__ __launch_bounds__(512) void k_router_mfma(int T, int d, int E,
                                                     const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     float* __restrict__ logits) {
  __shared__ float red[kRouterMfmaWaves][16][16 * NJ];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t0 = blockIdx.x * 16;
  const int eb = blockIdx.y * 16 * NJ;  // first expert of this block
  const int lr = lane % 16, kc = (lane / 16) * 8;
  const int steps = d / 32;
  const int s0 = wave * steps / kRouterMfmaWaves, s1 = (wave + 1) * steps / kRouterMfmaWaves;
  // rows past T or E are clamped (their results are discarded)
  const uint16_t* xr = x + (size_t)min(t0 + lr, T - 1) * d + kc;
  const uint16_t* wr[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) wr[j] = w + (size_t)min(eb + 16 * j + lr, E - 1) * d + kc;
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // K-steps in batches of U: all loads of a batch are issued before its first MFMA.  A tail
  // batch re-reads its last step and zeroes that step's activations, so the duplicate adds 0.
  constexpr int U = 4;
  const bf16x8 zero = {};
  for (int sb = s0; sb < s1; sb += U) {
    bf16x8 a[U], b[U][NJ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(sb + u, s1 - 1) * 32;
      a[u] = *reinterpret_cast<const bf16x8*>(xr + kk);
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[u][j] = *reinterpret_cast<const bf16x8*>(wr[j] + kk);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its MFMAs
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bf16x8 au = sb + u < s1 ? a[u] : zero;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, b[u][j], acc[j], 0, 0, 0);
    }
  }
  // lane holds tokens 4*(lane/16) + v of expert 16*j + lane%16
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][(lane / 16) * 4 + v][16 * j + lr] = acc[j][v];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 16 * NJ; i += blockDim.x) {
    const int tt = i / (16 * NJ), ej = i % (16 * NJ), e = eb + ej;
    if (t0 + tt < T && e < E) {
      const float sum = ((red[0][tt][ej] + red[1][tt][ej]) + (red[2][tt][ej] + red[3][tt][ej])) +
                        ((red[4][tt][ej] + red[5][tt][ej]) + (red[6][tt][ej] + red[7][tt][ej]));
      logits[(size_t)(t0 + tt) * E + e] = sum + (bias ? bias[e] : 0.f);
    }
  }
}

}  // namespace

namespace {

// grid: ceil(T / 4); block 256 (one wavefront per token)
__global__ __launch_bounds__(256) void k_topk(int T, int E, int k, int renorm,
                                              const float* __restrict__ logits,
                                              int32_t* __restrict__ ids, float* __restrict__ wout) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  float l[4];
  topk_load(logits + (size_t)t * E, E, lane, l);
  topk_select(l, E, k, renorm, lane, ids, wout, t, nullptr);
}

// 16-byte chunks of a row (8 bf16 or 4 fp32) as floats and back
template <typename AT> struct Chunk;
template <> struct Chunk<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& c, float (&f)[8]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_lo(w[q]);
      f[2 * q + 1] = bf16_hi(w[q]);
    }
  }
  __device__ static uint4 pack(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& c, float (&f)[4]) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  }
  __device__ static uint4 pack(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// y = x / sqrt(mean(x^2) + eps), one block per token, fp32 sums in a fixed order.  Rows are
// whole 16-byte chunks at 16-byte aligned addresses; each thread loads its (at most R) chunks
// once, keeps them in registers for the sum of squares and the scaling, and writes 16-byte
// stores.
template <typename AT, int R>
__global__ __launch_bounds__(256) void k_rmsnorm(int d, float eps, const AT* __restrict__ x,
                                                   AT* __restrict__ y) {
  using C = Chunk<AT>;
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int nc = d / C::N;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * d);
  uint4* yr = reinterpret_cast<uint4*>(y + (size_t)t * d);
  uint4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = threadIdx.x + 256 * r;
    v[r] = c < nc ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float f[C::N];
    C::unpack(v[r], f);
#pragma unroll
    for (int q = 0; q < C::N; ++q) ss = fmaf(f[q], f[q], ss);
  }
  ss = wave_sum_u(ss);
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = threadIdx.x + 256 * r;
    if (c < nc) {
      float f[C::N];
      C::unpack(v[r], f);
#pragma unroll
      for (int q = 0; q < C::N; ++q) f[q] *= inv;
      yr[c] = C::pack(f);
    }
  }
}

template <typename AT>
hipError_t rmsnorm_typed(int T, int d, const AT* x, AT* y, float eps, hipStream_t s) {
  constexpr int N = Chunk<AT>::N;
  const int per_thread = (d / N + 255) / 256;  // 16-byte chunks per thread
  // the descriptor and pointer checks guarantee d % 16 == 0, d <= 16384 and aligned rows
  if (d % N != 0 || (((uintptr_t)x | (uintptr_t)y) & 15) != 0 || per_thread > 16)
    return hipErrorInvalidValue;
  const int id = MOE_KERNEL_RMSNORM;
  if (per_thread <= 1) return launch(id, k_rmsnorm<AT, 1>, T, 256, 0, s, d, eps, x, y);
  if (per_thread <= 2) return launch(id, k_rmsnorm<AT, 2>, T, 256, 0, s, d, eps, x, y);
  if (per_thread <= 4) return launch(id, k_rmsnorm<AT, 4>, T, 256, 0, s, d, eps, x, y);
  if (per_thread <= 8) return launch(id, k_rmsnorm<AT, 8>, T, 256, 0, s, d, eps, x, y);
  return launch(id, k_rmsnorm<AT, 16>, T, 256, 0, s, d, eps, x, y);
}

}  // namespace

hipError_t launch_rmsnorm(const LayerDims& L, int T, const void* x, void* xn, float eps,
                          hipStream_t s) {
  if (L.act == MOE_F32) return rmsnorm_typed<float>(T, L.d, (const float*)x, (float*)xn, eps, s);
  return rmsnorm_typed<uint16_t>(T, L.d, (const uint16_t*)x, (uint16_t*)xn, eps, s);
}

// Matrix-core router: bf16, K in whole MFMA steps, past decode sizes.
static bool router_on_mfma(const LayerDims& L, int T) {
  return L.act == MOE_BF16 && L.d % 32 == 0 && T > kRouterMfmaMinT;
}

hipError_t launch_router_logits(const LayerDims& L, int T, const void* x, const void* w_router,
                                const float* bias, float* logits, hipStream_t s) {
  if (router_on_mfma(L, T)) {
    // one 16-expert tile per block (four times the blocks of one block per token group, so
    // the router reads spread over more CUs)
    const dim3 grid((T + 15) / 16, (L.E + 15) / 16);
    return launch(MOE_KERNEL_ROUTER, k_router_mfma<1>, grid, 512, 0, s, T, L.d, L.E,
                  (const uint16_t*)x, (const uint16_t*)w_router, bias, logits);
  }
  const int esz = L.act == MOE_F32 ? 4 : 2;
  int tb = kRouteTB;
  while (tb > 1 && (size_t)tb * L.d * esz > 64 * 1024) tb >>= 1;
  // decode sizes: one expert per wavefront, many blocks; otherwise all experts per block
  const int epw = (T <= 64) ? 1 : (L.E + 3) / 4;
  dim3 grid((T + tb - 1) / tb, (L.E + 4 * epw - 1) / (4 * epw));
  const size_t lds = (size_t)tb * L.d * esz;
  if (L.act == MOE_F32)
    return launch(MOE_KERNEL_ROUTER, k_router_logits<float>, grid, 256, lds, s, T, L.d, L.E, epw, tb,
                  (const float*)x, (const float*)w_router, bias, logits);
  return launch(MOE_KERNEL_ROUTER, k_router_logits<uint16_t>, grid, 256, lds, s, T, L.d, L.E, epw,
                tb, (const uint16_t*)x, (const uint16_t*)w_router, bias, logits);
}

hipError_t launch_topk(const LayerDims& L, int T, const float* logits, int32_t* ids, float* w,
                       hipStream_t s) {
  return launch(MOE_KERNEL_TOPK, k_topk, (T + 3) / 4, 256, 0, s, T, L.E, L.k, L.renorm, logits, ids, w);
}

}  // namespace moe
