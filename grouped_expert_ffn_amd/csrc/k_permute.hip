// Stable sort of the T*k (token, slot) rows by expert, with a block-wide prefix scan and no
// atomics (the switchyard page sorts rows by expert this way, §02 "Route and sort").
//
// One workgroup of 16 wavefronts.  The expert ids are first staged in LDS (every thread
// issues all of its loads before the first store, so the staging costs one memory round
// trip rather than one per step; the fused kernel writes them there from its top-k).
// Wavefront w owns a contiguous range of flat rows, walked 64 at a time.  Inside a step, lanes holding the same expert id find each other with eight
// ballots (one per bit of the id); the lowest such lane is the group's leader and the rank
// of a lane among its peers is a popcount of the lower peers.  Pass 1 builds a per-wavefront
// histogram in LDS (only leaders write, and no two leaders share an address), a column scan
// over wavefronts plus an exclusive scan over experts turns it into per-wavefront bases, and
// pass 2 repeats the walk and scatters each row to base + rank.  Because wavefronts own
// ascending ranges and lanes are ranked in order, rows of one expert keep ascending flat
// index: the sort is stable and its result unique.
//
// Past kSingleMaxRows rows the sort is spread over workgroups of kPermChunk rows each: a
// first kernel writes every chunk's expert histogram; each chunk's per-expert base (the rows
// of that expert in the chunks before it) and the expert totals come from summing the
// histograms, inside the sort kernel while there are few chunks, else by a scan launch; the
// sort kernel then runs once per chunk (the same offsets the one-workgroup kernel computes,
// so the result is identical).
//
// With a capacity limit C, a row whose place in its expert's segment is C or later is
// dropped (inv_perm = -1): the segment keeps ascending flat order, so these are the pairs
// that reached the expert after its first C.
//
// The sort kernel (its first workgroup) also writes the launch plan of the grouped FFN: the
// ascending list of groups that have rows (touched routed experts, then the shared experts)
// and, for the MFMA path, the list of (group, first row) M-tiles.
#include "moe_internal.h"
#include "small_sort.h"
#include "topk.h"

namespace moe {

namespace {

constexpr int kPermWaves = 16;
// T*k limit of the fused top-k + sort kernel.  Its one workgroup selects every token's top-k
// in turn (16 wavefronts), so past a few hundred rows the separate top-k launch (a wavefront
// per token over the whole chip) and the one-workgroup sort are faster: OLMoE layer -5% at
// T=64 (512 rows), -7% at 128, -12% at 256; DeepSeek -3% at 64, -6% at 128, -12% at 256;
// equal up to 256 rows (OLMoE T=32), where the fused launch saves a launch.
constexpr int kFusedMaxRows = 256;
constexpr int kSingleMaxRows = 4096;  // T*k up to which one workgroup sorts every row
constexpr int kDirectBaseChunks = 64;  // chunks up to which the sort blocks sum their own bases
constexpr int kStageLoads = kSingleMaxRows / (kPermWaves * kWave);  // staging loads per thread
static_assert(kFusedMaxRows <= kSingleMaxRows, "the fused kernel sorts in one workgroup");
static_assert(kPermChunk == kPermWaves * kWave, "one 64-row step per wavefront and chunk");

// FUSED: the kernel first runs top-k on `logits` for every token (one wavefront per token),
// writing ids/w to global memory and the ids to LDS, and then sorts from LDS.
template <bool FUSED>
__global__ __launch_bounds__(1024) void k_permute(int T, int k, int E, int S, int tile_m,
                                                  const float* __restrict__ logits, int renorm,
                                                  float* __restrict__ topk_w,
                                                  int32_t* __restrict__ ids,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm,
                                                  int32_t* __restrict__ inv_perm,
                                                  int32_t* __restrict__ plan,
                                                  const int32_t* __restrict__ chunk_hist,
                                                  int hist_scanned, int cap) {
  __shared__ int hist[kPermWaves][256];
  __shared__ int pre[kMaxGroups];
  __shared__ int seg[kMaxGroups];  // start of each expert's sorted segment
  __shared__ int cnt[kMaxGroups];
  __shared__ int base[kMaxGroups];
  __shared__ int touched[kMaxGroups];
  __shared__ int tile_start[kMaxGroups + 1];
  __shared__ int n_routed_touched;
  __shared__ int keys_lds[kSingleMaxRows];  // expert ids of rows r0..r1-1

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int N = T * k;
  // rows [r0, r1) of this workgroup: all of them, or chunk blockIdx.x of the multi-workgroup sort
  const bool multi = chunk_hist != nullptr;
  const int r0 = multi ? blockIdx.x * kPermChunk : 0;
  const int r1 = multi ? min(N, r0 + kPermChunk) : N;
  const int nrows = r1 - r0;
  const int per_wave = ((nrows + kPermWaves * kWave - 1) / (kPermWaves * kWave)) * kWave;
  const int begin = r0 + wave * per_wave, end = min(r1, begin + per_wave);
  const bool lead_block = blockIdx.x == 0;  // writes counts, offsets and the plan
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int e = lane; e < 256; e += kWave) hist[wave][e] = 0;
  if (FUSED) {
    // the next token's logits are loaded while the current token is selected
    float cur[4], nxt[4];
    if (wave < T) topk_load(logits + (size_t)wave * E, E, lane, cur);
    for (int t = wave; t < T; t += kPermWaves) {
      const int tn = t + kPermWaves;
      if (tn < T) topk_load(logits + (size_t)tn * E, E, lane, nxt);
      topk_select(cur, E, k, renorm, lane, ids, topk_w, t, keys_lds);
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    }
  } else {
    int v[kStageLoads];
#pragma unroll
    for (int j = 0; j < kStageLoads; ++j) {
      const int i = tid + j * kPermWaves * kWave;
      v[j] = i < nrows ? ids[r0 + i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kStageLoads; ++j) {
      const int i = tid + j * kPermWaves * kWave;
      if (i < nrows) keys_lds[i] = v[j];
    }
  }
  __syncthreads();
  auto key_of = [&](int f) { return keys_lds[f - r0]; };

  // pass 1: per-wavefront histograms
  for (int b0 = begin; b0 < end; b0 += kWave) {
    const int f = b0 + lane;
    const bool valid = f < end;
    int key = valid ? key_of(f) : 0;
    key = ((unsigned)key < (unsigned)E) ? key : E - 1;
    const uint64_t peers = peer_mask(key, valid);
    const int leader = __ffsll((long long)peers) - 1;
    if (valid && lane == leader) hist[wave][key] += __popcll(peers);
  }
  __syncthreads();

  // column scan over wavefronts; the expert totals (and, for a chunk, the rows of each expert
  // in the chunks before it) come from the chunk histograms in the multi-workgroup sort
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    if (multi) {
      const int nb = (N + kPermChunk - 1) / kPermChunk;
      if (hist_scanned) {
        // this chunk's base for each expert and the expert totals (k_perm_scan)
        pre[e] = chunk_hist[(size_t)blockIdx.x * E + e];
        cnt[e] = chunk_hist[(size_t)nb * E + e];
      } else {
        // few chunks: the rows of expert e in the chunks before this one, and in all of them,
        // summed here (loads in batches of 8 in flight) instead of by a scan launch
        int before = 0, total = 0;
        for (int b0 = 0; b0 < nb; b0 += 8) {
          int c[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) c[u] = b0 + u < nb ? chunk_hist[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            before += b0 + u < (int)blockIdx.x ? c[u] : 0;
            total += c[u];
          }
        }
        pre[e] = before;
        cnt[e] = total;
      }
    } else {
      pre[e] = 0;
      cnt[e] = run;
    }
  }
  __syncthreads();

  // exclusive scans over experts (row offsets, touched-list positions): wavefront 0,
  // four experts per lane
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
        base[e] = ex + pre[e];
        seg[e] = ex;
        if (lead_block) {
          counts[e] = c[i];
          offsets[e] = ex;
        }
        if (c[i] > 0) touched[exf++] = e;
        ex += c[i];
      }
    }
    if (lane == kWave - 1) n_routed_touched = inclf;
    if (lead_block && lane <= S) offsets[E + lane] = N + lane * T;
  }
  __syncthreads();

  const int nrt = n_routed_touched;
  const int n_groups = nrt + S;
  if (tid < S) touched[nrt + tid] = E + tid;
  // per-wavefront bases
  for (int e = tid; e < E; e += blockDim.x) {
    const int b = base[e];
    for (int w = 0; w < kPermWaves; ++w) hist[w][e] += b;
  }
  __syncthreads();

  // pass 2: scatter
  for (int b0 = begin; b0 < end; b0 += kWave) {
    const int f = b0 + lane;
    const bool valid = f < end;
    int key = valid ? key_of(f) : 0;
    key = ((unsigned)key < (unsigned)E) ? key : E - 1;
    const uint64_t peers = peer_mask(key, valid);
    const int leader = __ffsll((long long)peers) - 1;
    const int pos = hist[wave][key] + __popcll(peers & lt_mask);
    if (valid) {
      perm[pos] = f;
      // with a capacity limit, rows past the first cap of the expert's segment are dropped
      inv_perm[f] = (cap == 0 || pos - seg[key] < cap) ? pos : -1;
    }
    if (valid && lane == leader) hist[wave][key] = hist[wave][key] + __popcll(peers);
  }

  // plan: touched groups and M-tiles (first workgroup only)
  if (!lead_block) return;
  int32_t* tl = plan + kPlanHeader;
  for (int i = tid; i < n_groups; i += blockDim.x) tl[i] = touched[i];
  if (tile_m > 0) {
    if (wave == 0) {
      // exclusive scan of tiles per touched group, five groups per lane
      int nt[5], s = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int p = 5 * lane + i;
        int rows = 0;
        if (p < n_groups) {
          const int g = touched[p];
          rows = g < E ? (cap ? min(cnt[g], cap) : cnt[g]) : T;
        }
        nt[i] = (rows + tile_m - 1) / tile_m;
        s += nt[i];
      }
      const int incl = wave_incl_scan(s, lane);
      int ex = incl - s;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int p = 5 * lane + i;
        if (p < kMaxGroups) tile_start[p] = ex;
        ex += nt[i];
      }
      if (lane == kWave - 1) tile_start[kMaxGroups] = incl;
    }
    __syncthreads();
    int32_t* tiles = tl + (E + S);
    for (int p = tid; p < n_groups; p += blockDim.x) {
      const int g = touched[p];
      const int rows = g < E ? (cap ? min(cnt[g], cap) : cnt[g]) : T;
      int o = tile_start[p];
      for (int m0 = 0; m0 < rows; m0 += tile_m, ++o) {
        tiles[2 * o] = g;
        tiles[2 * o + 1] = m0;
      }
    }
    if (tid == 0) plan[1] = tile_start[kMaxGroups];
  } else if (tid == 0) {
    plan[1] = 0;
  }
  if (tid == 0) {
    plan[0] = n_groups;
    plan[2] = tile_m;
    plan[3] = cap;
  }
}

// Expert histogram of each chunk of kPermChunk rows (one 64-row step per wavefront), summed
// over the wavefronts in a fixed order.  grid: ceil(T*k / kPermChunk); block 1024
__global__ __launch_bounds__(1024) void k_perm_hist(int N, int E, const int32_t* __restrict__ ids,
                                                    int32_t* __restrict__ chunk_hist) {
  __shared__ int hist[kPermWaves][256];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int e = lane; e < 256; e += kWave) hist[wave][e] = 0;
  const int f = blockIdx.x * kPermChunk + tid;
  const bool valid = f < N;
  int key = valid ? ids[f] : 0;
  key = ((unsigned)key < (unsigned)E) ? key : E - 1;
  __syncthreads();
  const uint64_t peers = peer_mask(key, valid);
  const int leader = __ffsll((long long)peers) - 1;
  if (valid && lane == leader) hist[wave][key] += __popcll(peers);
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) run += hist[w][e];
    chunk_hist[(size_t)blockIdx.x * E + e] = run;
  }
}

// Exclusive scan of the chunk histograms over chunks, in place, one expert per thread; the
// expert totals go after the last chunk.  grid: ceil(E / 256); block 256
__global__ __launch_bounds__(256) void k_perm_scan(int nb, int E, int32_t* __restrict__ chunk_hist) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  int run = 0;
  for (int b = 0; b < nb; ++b) {
    const int c = chunk_hist[(size_t)b * E + e];
    chunk_hist[(size_t)b * E + e] = run;
    run += c;
  }
  chunk_hist[(size_t)nb * E + e] = run;
}

// Up to 64 rows: the one-wavefront sort (with the top-k first when logits are given; 16
// wavefronts select up to 16 tokens at once).  grid: 1; block 1024
__global__ __launch_bounds__(1024) void k_permute_small(const SortArgs p) { small_topk_sort(p); }

}  // namespace

hipError_t launch_permute(const LayerDims& L, int T, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* plan,
                          int tile_m, hipStream_t s) {
  const int N = T * L.k;
  int32_t* idsm = const_cast<int32_t*>(ids);
  if (N <= kSmallSortRows) {
    const SortArgs p{T, L.k, L.E, L.S, tile_m, L.renorm, capacity_rows(L, T), nullptr, nullptr, idsm,
                     counts, offsets, perm, inv_perm, plan};
    return launch(MOE_KERNEL_PERMUTE, k_permute_small, 1, 1024, 0, s, p);
  }
  if (N <= kSingleMaxRows)
    return launch(MOE_KERNEL_PERMUTE, k_permute<false>, 1, 1024, 0, s, T, L.k, L.E, L.S, tile_m,
                  nullptr, 0, nullptr, idsm, counts, offsets, perm, inv_perm, plan, nullptr, 0,
                  capacity_rows(L, T));
  // two or three launches: the timer records its start before the first and its stop after
  // the last launch made while it is alive
  LaunchTimer timer(MOE_KERNEL_PERMUTE, s);
  int32_t* chunk_hist = plan + plan_hist_offset(T, L.k, L.E, L.S);
  const int nb = (N + kPermChunk - 1) / kPermChunk;
  k_perm_hist<<<nb, 1024, 0, s>>>(N, L.E, ids, chunk_hist);
  // up to kDirectBaseChunks chunks each sort block sums the histograms before it itself (at
  // most that many loads per expert); beyond, one scan launch does it once for all blocks
  const int scanned = nb > kDirectBaseChunks;
  if (scanned) k_perm_scan<<<(L.E + 255) / 256, 256, 0, s>>>(nb, L.E, chunk_hist);
  k_permute<false><<<nb, 1024, 0, s>>>(T, L.k, L.E, L.S, tile_m, nullptr, 0, nullptr, idsm, counts,
                                       offsets, perm, inv_perm, plan, chunk_hist, scanned,
                                       capacity_rows(L, T));
  return hipGetLastError();
}

bool topk_permute_fusable(const LayerDims& L, int T) { return (size_t)T * L.k <= kFusedMaxRows; }

hipError_t launch_topk_permute(const LayerDims& L, int T, const float* logits, int32_t* ids,
                               float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv_perm, int32_t* plan, int tile_m, hipStream_t s) {
  if ((size_t)T * L.k <= kSmallSortRows) {
    const SortArgs p{T, L.k, L.E, L.S, tile_m, L.renorm, capacity_rows(L, T), logits, topk_w, ids,
                     counts, offsets, perm, inv_perm, plan};
    return launch(MOE_KERNEL_PERMUTE, k_permute_small, 1, 1024, 0, s, p);
  }
  return launch(MOE_KERNEL_PERMUTE, k_permute<true>, 1, 1024, 0, s, T, L.k, L.E, L.S, tile_m, logits,
                L.renorm, topk_w, ids, counts, offsets, perm, inv_perm, plan, nullptr, 0,
                capacity_rows(L, T));
}

}  // namespace moe
