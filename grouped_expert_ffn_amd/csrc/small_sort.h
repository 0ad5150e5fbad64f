// Top-k and the stable sort by expert for up to one wavefront of rows (T*k <= 64), in one
// block of 4-16 wavefronts: the decode-size form of the sort kernel (same result, the unique
// stable order), callable from a kernel whose other blocks do other work.
//
// The wavefronts select the tokens' top-k (one token per wavefront at a time) into LDS;
// then one wavefront holds row f in lane f.  Lanes with the same expert find each other with
// eight ballots (one per bit of the id); the lowest is the group's leader and writes the
// group's size, and a lane's rank among its peers is a popcount of the lower peers.  One
// exclusive scan over the experts (four per lane) gives every expert's segment start, the
// touched-group list and the counts; a row's place is its segment start plus its rank.  There
// are no per-wavefront histograms to combine, so the whole sort is three short steps between
// workgroup barriers.
#pragma once

#include "moe_internal.h"
#include "topk.h"

namespace moe {

constexpr int kMaxGroups = 256 + 8;  // routed experts + shared experts, at the limits

// Inclusive prefix sum over the wavefront's 64 lanes (all active): a Hillis-Steele scan
// inside each row of 16 lanes by DPP row shifts (a lane with no source lane adds 0), then
// each row adds the totals of the rows before it, read from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
}

// Lanes whose (valid) 8-bit key equals this lane's, as a 64-bit mask.
__device__ __forceinline__ uint64_t peer_mask(int key, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

struct SortArgs {
  int T, k, E, S, tile_m, renorm, cap;
  const float* logits;  // the top-k of these logits first, or null: ids are given
  float* topk_w;
  int32_t* ids;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* plan;
};

// Every thread of the block calls this (it holds workgroup barriers); T * k <= 64; the block
// is 256-1024 threads.
__device__ __forceinline__ void small_topk_sort(const SortArgs& p) {
  __shared__ int keys[kSmallSortRows];
  __shared__ int cnt[kMaxGroups];
  __shared__ int seg[kMaxGroups];
  __shared__ int touched[kMaxGroups];
  __shared__ int n_routed;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int nw = blockDim.x / kWave;
  const int T = p.T, k = p.k, E = p.E, S = p.S;
  const int N = T * k;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  if (p.logits) {
    // one token per wavefront at a time; the next token's logits load during the selection
    float cur[4], nxt[4];
    if (wave < T) topk_load(p.logits + (size_t)wave * E, E, lane, cur);
    for (int t = wave; t < T; t += nw) {
      const int tn = t + nw;
      if (tn < T) topk_load(p.logits + (size_t)tn * E, E, lane, nxt);
      topk_select(cur, E, k, p.renorm, lane, p.ids, p.topk_w, t, keys);
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
  } else if (tid < N) {
    keys[tid] = p.ids[tid];
  }
  __syncthreads();

  // (1) lane f holds row f: peers, rank among them, group sizes
  const bool valid = wave == 0 && lane < N;
  int key = valid ? keys[lane] : 0;
  key = ((unsigned)key < (unsigned)E) ? key : E - 1;
  int before = 0;
  if (wave == 0) {
    const uint64_t peers = peer_mask(key, valid);
    const int leader = __ffsll((long long)peers) - 1;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    before = __popcll(peers & lt_mask);
    if (valid && lane == leader) cnt[key] = __popcll(peers);
  }
  __syncthreads();

  // (2) exclusive scans over the experts (segment starts, touched-list positions), four
  //     experts per lane
  if (wave == 0) {
    int c[4], s = 0, sf = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? cnt[e] : 0;
      s += c[i];
      sf += c[i] > 0;
    }
    const int incl = wave_incl_scan(s, lane), inclf = wave_incl_scan(sf, lane);
    int ex = incl - s, exf = inclf - sf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        seg[e] = ex;
        p.counts[e] = c[i];
        p.offsets[e] = ex;
        if (c[i] > 0) touched[exf++] = e;
        ex += c[i];
      }
    }
    if (lane == kWave - 1) n_routed = inclf;
    if (lane <= S) p.offsets[E + lane] = N + lane * T;
  }
  __syncthreads();

  // (3) scatter, and the launch plan: touched groups (routed, then shared) and, for the
  //     GEMM, the (group, first row) M-tiles
  if (wave != 0) return;
  if (valid) {
    const int pos = seg[key] + before;
    p.perm[pos] = lane;
    p.inv_perm[lane] = (p.cap == 0 || before < p.cap) ? pos : -1;
  }
  const int nrt = n_routed;
  const int n_groups = nrt + S;  // at most 64 + 8
  int32_t* tl = p.plan + kPlanHeader;
  int grp[2], rows[2], nt[2], tsum = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // groups 2 * lane and 2 * lane + 1
    const int q = 2 * lane + i;
    grp[i] = q < nrt ? touched[q] : E + (q - nrt);
    rows[i] = 0;
    if (q < n_groups) {
      tl[q] = grp[i];
      rows[i] = q < nrt ? (p.cap ? min(cnt[grp[i]], p.cap) : cnt[grp[i]]) : T;
    }
    nt[i] = p.tile_m > 0 ? (rows[i] + p.tile_m - 1) / p.tile_m : 0;
    tsum += nt[i];
  }
  const int tincl = wave_incl_scan(tsum, lane);
  if (p.tile_m > 0) {
    int32_t* tiles = tl + (E + S);
    int o = tincl - tsum;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      for (int m0 = 0; m0 < rows[i]; m0 += p.tile_m, ++o) {
        tiles[2 * o] = grp[i];
        tiles[2 * o + 1] = m0;
      }
  }
  if (lane == kWave - 1) {
    p.plan[0] = n_groups;
    p.plan[1] = tincl;
    p.plan[2] = p.tile_m;
    p.plan[3] = p.cap;
  }
}

}  // namespace moe
