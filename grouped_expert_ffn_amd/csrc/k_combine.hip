// Deterministic combine back to token order (switchyard page, hero statistics: expert-
// parallel output equal to one GPU bit for bit; §02 "Kernels and dispatch": no atomics).
// Every output element is owned by one thread, which reads the token's k routed rows
// through inv_perm, then its shared-expert rows, then the residual, and sums them in fp32
// in exactly that order before a single rounding.  Loads and stores are 16 bytes per lane,
// and each thread has its rows' loads in flight together rather than one round trip per row.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kSlotBatch = 8;  // routed rows in flight per thread
constexpr int kMaxShared = 8;  // the descriptor's limit on shared experts

template <typename AT>
__global__ __launch_bounds__(256) void k_combine(int T, int d, int k, int S,
                                                 const AT* __restrict__ rows,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ w,
                                                 const AT* residual, AT* y) {
  constexpr int V = 16 / sizeof(AT);
  const int t = blockIdx.x;
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * V;
  if (c >= d) return;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  auto add = [&](const uint4& v, float wt, bool scaled) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    if (sizeof(AT) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = bf16_lo(u[i]), hi = bf16_hi(u[i]);
        acc[2 * i] = scaled ? fmaf(wt, lo, acc[2 * i]) : acc[2 * i] + lo;
        acc[2 * i + 1] = scaled ? fmaf(wt, hi, acc[2 * i + 1]) : acc[2 * i + 1] + hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = __uint_as_float(u[i]);
        acc[i] = scaled ? fmaf(wt, f, acc[i]) : acc[i] + f;
      }
    }
  };
  auto load = [&](const AT* src) { return *reinterpret_cast<const uint4*>(src); };
  // routed rows, eight slots at a time: the batch's loads are all in flight before the first
  // is summed (a dropped slot, inv_perm < 0, reads row 0 and is skipped), then the sums run
  // in slot order
  for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
    uint4 v[kSlotBatch];
    int r[kSlotBatch];
    float wt[kSlotBatch];
    // the batch's row indices and weights (whole batches as unconditional loads, which the
    // compiler merges into wide scalar loads)
    const bool full = j0 + kSlotBatch <= k;
#pragma unroll
    for (int u = 0; u < kSlotBatch; ++u) {
      const size_t i = (size_t)t * k + (full ? j0 + u : min(j0 + u, k - 1));
      r[u] = (full || j0 + u < k) ? inv_perm[i] : -1;
      wt[u] = w[i];
    }
#pragma unroll
    for (int u = 0; u < kSlotBatch; ++u) v[u] = load(rows + (size_t)(r[u] < 0 ? 0 : r[u]) * d + c);
#pragma unroll
    for (int u = 0; u < kSlotBatch; ++u)
      if (r[u] >= 0) add(v[u], wt[u], true);
  }
  // shared-expert rows and the residual, loaded together, summed in that order
  uint4 vs[kMaxShared + 1];
#pragma unroll
  for (int s = 0; s < kMaxShared; ++s)
    if (s < S) vs[s] = load(rows + ((size_t)T * k + (size_t)s * T + t) * d + c);
  if (residual) vs[kMaxShared] = load(residual + (size_t)t * d + c);
#pragma unroll
  for (int s = 0; s < kMaxShared; ++s)
    if (s < S) add(vs[s], 1.f, false);
  if (residual) add(vs[kMaxShared], 1.f, false);
  AT* dst = y + (size_t)t * d + c;
  if (sizeof(AT) == 2) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(dst) = o;
  } else {
    *reinterpret_cast<uint4*>(dst) =
        make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                   __float_as_uint(acc[3]));
  }
}

}  // namespace

hipError_t launch_combine(const LayerDims& L, int T, const void* rows, const int32_t* inv_perm,
                          const float* topk_w, const void* residual, void* y, hipStream_t s) {
  const int V = L.act == MOE_F32 ? 4 : 8;
  const int per_block = 256 * V;
  dim3 grid(T, (L.d + per_block - 1) / per_block);
  if (L.act == MOE_F32)
    return launch(MOE_KERNEL_COMBINE, k_combine<float>, grid, 256, 0, s, T, L.d, L.k, L.S,
                  (const float*)rows, inv_perm, topk_w, (const float*)residual, (float*)y);
  return launch(MOE_KERNEL_COMBINE, k_combine<uint16_t>, grid, 256, 0, s, T, L.d, L.k, L.S,
                (const uint16_t*)rows, inv_perm, topk_w, (const uint16_t*)residual, (uint16_t*)y);
}

}  // namespace moe
