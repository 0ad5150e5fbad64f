// Top-k gating of one token by one wavefront; shared by the top-k and fused permute kernels.
//
// Lane l holds the logits of experts l, l+64, l+128 and l+192 (E <= 256), each with an
// order-preserving 32-bit code (NaN lowest).  Up to 64 experts the wavefront sorts the keys
// (code, 255 - expert) with a 21-step bitonic network and lane r holds slot r.  Beyond, the
// k slots are filled in k rounds: every lane offers its best remaining expert (highest code,
// then lowest id), a wave-wide max over the offers picks the code, a wave-wide min over the
// lanes offering that code picks the lowest id, and that expert leaves the pool.  Either way
// slots are ordered by descending logit, equal logits go to the lower expert id, and NaN
// ranks below every number.
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

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t readlane_u(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
// wave-wide max / min of uint32, the same in every lane (all 64 lanes must be active)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  return max(max(readlane_u(v, 0), readlane_u(v, 16)), max(readlane_u(v, 32), readlane_u(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<0xB1>(v));
  v = min(v, dpp_u<0x4E>(v));
  v = min(v, dpp_u<0x141>(v));
  v = min(v, dpp_u<0x140>(v));
  return min(min(readlane_u(v, 0), readlane_u(v, 16)), min(readlane_u(v, 32), readlane_u(v, 48)));
}

// The token's logits into the lane's four slots (-inf past E).  All four loads are issued
// unconditionally (clamped to the row), so they are in flight together.
__device__ __forceinline__ void topk_load(const float* __restrict__ lrow, int E, int lane, float (&l)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    const float v = lrow[min(e, E - 1)];
    l[i] = e < E ? v : -INFINITY;
  }
}

// inverse of order_bits (NaN comes back as a NaN, -0 as +0)
__device__ __forceinline__ float from_order_bits(uint32_t c) {
  return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

// the value of lane ^ STRIDE (STRIDE a power of two below 64)
template <int STRIDE>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (STRIDE == 1) {
    return dpp_u<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (STRIDE == 2) {
    return dpp_u<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (STRIDE < 32) {
    // ds_swizzle bit mode within 32 lanes: and-mask 0x1F, or-mask 0, xor-mask STRIDE
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (STRIDE << 10));
  } else {
    return (uint32_t)__shfl_xor((int)v, 32, kWave);
  }
}

// one compare-exchange of a bitonic network over the wavefront (blocks of SIZE lanes, pairs
// STRIDE apart): the lane keeps the larger key where the final order is descending
template <int STRIDE, int SIZE>
__device__ __forceinline__ uint64_t bitonic_cx(uint64_t key, int lane) {
  const uint64_t other = ((uint64_t)xor_lane<STRIDE>((uint32_t)(key >> 32)) << 32) |
                         xor_lane<STRIDE>((uint32_t)key);
  const bool keep_max = ((lane & SIZE) == 0) == ((lane & STRIDE) == 0);
  return keep_max == (key > other) ? key : other;
}

// the lanes' 64-bit keys sorted in descending order, lane 0 holding the largest
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key, int lane) {
  key = bitonic_cx<1, 2>(key, lane);
  key = bitonic_cx<2, 4>(key, lane);
  key = bitonic_cx<1, 4>(key, lane);
  key = bitonic_cx<4, 8>(key, lane);
  key = bitonic_cx<2, 8>(key, lane);
  key = bitonic_cx<1, 8>(key, lane);
  key = bitonic_cx<8, 16>(key, lane);
  key = bitonic_cx<4, 16>(key, lane);
  key = bitonic_cx<2, 16>(key, lane);
  key = bitonic_cx<1, 16>(key, lane);
  key = bitonic_cx<16, 32>(key, lane);
  key = bitonic_cx<8, 32>(key, lane);
  key = bitonic_cx<4, 32>(key, lane);
  key = bitonic_cx<2, 32>(key, lane);
  key = bitonic_cx<1, 32>(key, lane);
  key = bitonic_cx<32, 64>(key, lane);
  key = bitonic_cx<16, 64>(key, lane);
  key = bitonic_cx<8, 64>(key, lane);
  key = bitonic_cx<4, 64>(key, lane);
  key = bitonic_cx<2, 64>(key, lane);
  key = bitonic_cx<1, 64>(key, lane);
  return key;
}

// Top-k for E <= 64 (one logit per lane), with the same result as the k rounds below: the
// keys (code, 255 - expert) are sorted across the wavefront, so lane r holds slot r
// (descending logit, the lower expert first among equal codes, NaN last); a lane's expert is
// chosen when its key is at least the k-th largest.  The softmax sums run over the same
// lanes in the same order as below, and a slot's weight is recomputed from its exactly
// recovered logit, so the outputs are identical.
__device__ __forceinline__ void topk_select_wave(const float (&l)[4], int E, int k, int renorm,
                                                 int lane, int32_t* __restrict__ ids,
                                                 float* __restrict__ wout, int t, int* keys_lds) {
  const bool valid = lane < E;
  const uint64_t key =
      valid ? (((uint64_t)order_bits(l[0]) << 32) | (uint32_t)(255 - lane)) : 0ull;
  const uint64_t top = wave_sort_desc(key, lane);
  const uint64_t kth = ((uint64_t)readlane_u((uint32_t)(top >> 32), k - 1) << 32) |
                       readlane_u((uint32_t)top, k - 1);
  const float m = wave_max_u(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
  const float z = valid ? expf(l[0] - m) : 0.f;
  const float zsum = wave_sum_u(z);
  const float den = renorm ? wave_sum_u((valid && key >= kth) ? z : 0.f) : zsum;
  if (lane < k) {
    const int e = 255 - (int)(uint32_t)top;
    const float zt = expf(from_order_bits((uint32_t)(top >> 32)) - m);
    ids[(size_t)t * k + lane] = e;
    wout[(size_t)t * k + lane] = zt / den;
    if (keys_lds) keys_lds[t * k + lane] = e;
  }
}

// Top-k gating of token t from its loaded logits, by one whole wavefront (all 64 lanes
// active).  Writes ids/w of the token's k slots; when keys_lds is given, the ids are also
// written there at t*k + slot.
__device__ __forceinline__ void topk_select(const float (&l)[4], int E, int k, int renorm, int lane,
                                            int32_t* __restrict__ ids, float* __restrict__ wout, int t,
                                            int* keys_lds) {
  if (E <= kWave) return topk_select_wave(l, E, k, renorm, lane, ids, wout, t, keys_lds);
  const int slots = (E + kWave - 1) / kWave;
  uint32_t code[4];
  bool live[4];
  int rank[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    code[i] = order_bits(l[i]);
    live[i] = lane + kWave * i < E;
    rank[i] = k;  // k = not chosen
  }
  for (int r = 0; r < k; ++r) {
    uint32_t bc = 0u, be = 0xFFFFu;
    bool any = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < slots && live[i] && (!any || code[i] > bc)) {  // later slots have higher ids
        bc = code[i];
        be = (uint32_t)(lane + kWave * i);
        any = true;
      }
    }
    const uint32_t m = wave_max_u32(any ? bc : 0u);
    const int win = (int)wave_min_u32((any && bc == m) ? be : 0xFFFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < slots && live[i] && lane + kWave * i == win) {
        live[i] = false;
        rank[i] = r;
      }
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
