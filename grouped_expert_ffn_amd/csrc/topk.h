// Top-k gating of one token by one wavefront; shared by the top-k and fused permute kernels.
#pragma once

#include "moe_internal.h"

namespace moe {

// order-preserving map of fp32 onto uint32 (+0 and -0 equal, NaN lowest)
__device__ __forceinline__ uint32_t order_bits(float v) {
  if (v != v) return 0u;
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Top-k gating of token t by one whole wavefront (all 64 lanes active).  Writes ids/w of
// the token's k slots; when keys_lds is given, the ids are also written there at t*k + slot.
__device__ __forceinline__ void topk_token(const float* __restrict__ lrow, int E, int k, int renorm, int lane,
                           int32_t* __restrict__ ids, float* __restrict__ wout, int t,
                           int* keys_lds) {
  float l[4];
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      l[i] = lrow[e];
      key[i] = ((uint64_t)order_bits(l[i]) << 32) | (uint32_t)(0xFFFFu - (uint32_t)e);
    } else {
      l[i] = -INFINITY;
      key[i] = 0;
    }
  }
  // rank of each key among the E keys
  int rank[4] = {0, 0, 0, 0};
  const int groups = (E + kWave - 1) / kWave;
  for (int j = 0; j < groups; ++j) {
    const int n_src = min(kWave, E - kWave * j);
    uint64_t kj = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) kj = (j == i) ? key[i] : kj;
    for (int src = 0; src < n_src; ++src) {
      const uint64_t other = readlane64(kj, src);
#pragma unroll
      for (int i = 0; i < 4; ++i) rank[i] += other > key[i];
    }
  }
  // softmax over all E, then the k chosen weights (optionally renormalised)
  const float m = wave_max_u(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
  float z[4], zs = 0.f, zsel = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool valid = lane + kWave * i < E;
    z[i] = valid ? expf(l[i] - m) : 0.f;
    zs += z[i];
    zsel += (valid && rank[i] < k) ? z[i] : 0.f;
  }
  const float zsum = wave_sum_u(zs);
  const float den = renorm ? wave_sum_u(zsel) : zsum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    if (e < E && rank[i] < k) {
      ids[(size_t)t * k + rank[i]] = e;
      wout[(size_t)t * k + rank[i]] = z[i] / den;
      if (keys_lds) keys_lds[t * k + rank[i]] = e;
    }
  }
}

}  // namespace moe
