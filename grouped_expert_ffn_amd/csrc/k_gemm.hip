// Grouped GEMM on the matrix cores for prefill sizes: every expert in one launch.
//
// The switchyard page runs all experts' GEMMs in one launch with the SwiGLU fused into the
// epilogue (§02 "One launch for all experts"); here that is one launch per matrix pair on
// gfx950's v_mfma_f32_16x16x32_bf16.  Work items come from the launch plan written by the
// permute kernel: each workgroup maps to one (M-tile, N-tile) of one group, in an XCD-aware
// order; work past the plan's count exits at once, so the grid can be sized from T*k
// without reading counts back to the host.  With a capacity limit in the plan, a routed
// group counts only its first C rows.
//
// Both kernels use 128-row M-tiles.  For gate/up an N-tile holds n gate channels followed by
// the same n up channels, and every wavefront holds matching gate and up accumulators, so
// silu(g)*u is formed in registers.  A rows are gathered through perm (token rows of x) or
// read in order (h rows).  128 rows keep the padding of the last tile of each expert small
// under skewed routing, where most experts get a few hundred rows.
//
//  * k_gemm_ring (bf16 or int8 weights, K a multiple of 32): 128x256 tiles, or 128x128 where
//    a tuned rule picks them (ring_tile_n below).  Four wavefronts side by side each own all
//    128 rows and a quarter of the columns, so a group's last, partly filled tile skips the
//    MFMAs of its empty 16-row slices in every wavefront alike.  The weights are
//    the first MFMA operand, which leaves 4 consecutive output channels in each lane for
//    8-byte stores.  BK=32 and a ring of NST LDS stages filled directly from global memory
//    by global_load_lds_dwordx4, issued NST-1 stages ahead of the MFMAs, so several stages
//    of loads are always in flight without holding registers.  The DMA writes lane l's 16
//    bytes at base + 16*l, so a stage is row-major (64-byte bf16 rows; 32-byte int8 weight
//    rows); the XOR swizzle that keeps the MFMA operand reads free of bank conflicts is
//    applied on the source side (each lane fetches a permuted 16-byte piece of its row).
//    int8 weights are widened to bf16 (exact) as they are read from LDS, and the
//    per-channel scales multiply the fp32 sums in the epilogue.
//  * k_gemm_ring64 (bf16 or int8 weights, K a multiple of 64): the ring kernel's tiles,
//    wavefronts and epilogue, with the weights staged 64 K deep in two slots (a bf16 row's
//    block is 128 bytes, a whole cache line, so a DMA instruction covers 8 full lines instead
//    of 16 half lines; an int8 row's block is 64 bytes, half lines instead of quarter lines)
//    and the activations 32 K deep in two slots.  Used whenever K allows; k_gemm_ring serves
//    K % 64 == 32.
//  * k_gemm (any K that is a multiple of 16): 128x128 tiles, four wavefronts in a 2x2 layout
//    each owning 64x64.  BK=64, LDS double buffer (rows padded by 16 bytes) with a register
//    prefetch of the next K-step; int8 weights are widened to bf16 on the way into LDS.
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128;
constexpr int THREADS = 256;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, each with its own L2

// general kernel
constexpr int BK = 64;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row
constexpr int A_ELEMS = BM * PITCH, B_ELEMS = BN * PITCH;
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
constexpr size_t GEMM_LDS = 2 * STAGE_ELEMS * sizeof(uint16_t);

// ring kernel
constexpr int RBK = 32;  // K elements per stage
constexpr int kRing128 = 3;  // ring depth of the 128-wide tile (the 256-wide one: 3)

struct GemmArgs {
  const void* in;   // gate/up: x [T, K] (gathered through perm); down: h [R, K]
  const void* w0;   // [G, N, K]: gate or down
  const void* w1;   // up
  const float* s0;
  const float* s1;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* plan;
  void* out;        // [R, N]
  int K, N, k, E, max_groups;
  int n_blk;        // output channels per N-tile (half the tile width for gate/up, all of it for down)
};

struct Work {
  int g, r0, M, m0, n0;
};

// XCD-aware work order.  Workgroups are dispatched round-robin over the 8 XCDs, so workgroup
// w runs on XCD w % 8.  XCD x takes a contiguous slice of the logical order (group, N-tile,
// M-tile): the M-tiles sharing a weight tile, and the N-tiles sharing a group's activation
// rows, run on the same L2 at about the same time.  The slice size comes from the plan's
// tile count, so every XCD gets valid work.  Returns false for a workgroup with no work.
template <int TBM>
__device__ __forceinline__ bool map_work_t(const GemmArgs& a, Work& w) {
  const int32_t* plan = a.plan;
  const int NT = (a.N + a.n_blk - 1) / a.n_blk;  // N-tiles per group
  const int valid = plan[1] * NT;
  const int per_xcd = (valid + kXcds - 1) / kXcds;
  const int wid = blockIdx.x;
  const int L = (wid % kXcds) * per_xcd + wid / kXcds;
  if (wid / kXcds >= per_xcd || L >= valid) return false;
  const int32_t* tiles = plan + kPlanHeader + a.max_groups;
  const int p = L / NT;  // a tile of the group that owns L
  w.g = tiles[2 * p];
  w.r0 = a.offsets[w.g];
  w.M = a.offsets[w.g + 1] - w.r0;
  if (w.g < a.E && plan[3] > 0) w.M = min(w.M, plan[3]);  // capacity: the rest is dropped
  const int mt = (w.M + TBM - 1) / TBM;           // the group's M-tiles
  const int first = p - tiles[2 * p + 1] / TBM;   // the group's first tile in the list
  const int o = L - first * NT;                   // position inside the group's (N, M) block
  w.m0 = (o % mt) * TBM;
  w.n0 = (o / mt) * a.n_blk;
  return true;
}

// Row of the A operand for M-tile row m (clamped into the group; results discarded).
// MODE 0 (gate/up) gathers token rows of x: through perm for a routed expert, row m itself
// for a shared expert (which sees every token in order).  MODE 1 (down) reads h row r0 + m.
template <int MODE>
__device__ __forceinline__ const uint16_t* a_row_t(const GemmArgs& a, const Work& w, int m) {
  m = min(m, w.M - 1);
  const int r = w.r0 + m;
  size_t src;
  if (MODE == 0)
    src = (w.g < a.E) ? (size_t)(a.perm[r] / a.k) : (size_t)m;
  else
    src = (size_t)r;
  return reinterpret_cast<const uint16_t*>(a.in) + src * a.K;
}

// Weight row (output channel) for B-tile row `row` (clamped into the matrix).
template <int MODE, int TBN>
__device__ __forceinline__ const unsigned char* b_row_t(const GemmArgs& a, const Work& w, int row,
                                                        int esz) {
  int n;
  const void* base;
  if (MODE == 0) {
    n = w.n0 + (row % (TBN / 2));
    base = row < TBN / 2 ? a.w0 : a.w1;
  } else {
    n = w.n0 + row;
    base = a.w0;
  }
  n = min(n, a.N - 1);
  return reinterpret_cast<const unsigned char*>(base) + ((size_t)w.g * a.N + n) * a.K * esz;
}

// The four B-tile rows a lane feeds to its wavefront's MFMAs (j = 0..3).
template <int MODE>
__device__ __forceinline__ int b_frag_row(int wn, int j, int lr) {
  if (MODE == 0)  // j = 0,1: gate channels; j = 2,3: the same up channels
    return (j < 2 ? 0 : BN / 2) + wn * 32 + (j % 2) * 16 + lr;
  return wn * 64 + j * 16 + lr;
}

// Epilogue: lane holds rows 4*(lane/16) + v, column lane%16 of each 16x16 tile.
template <int MODE, bool I8>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const Work& w, int wm, int wn,
                                           int lane, const f32x4 (&acc)[4][4]) {
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const int N = a.N, lr = lane % 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = w.m0 + wm * 64 + i * 16 + (lane / 16) * 4 + v;
      if (m >= w.M) continue;
      const size_t orow = (size_t)(w.r0 + m) * N;
      if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = w.n0 + wn * 32 + j * 16 + lr;
          if (n < N) {
            float gv = acc[i][j][v], uv = acc[i][j + 2][v];
            if (I8) {
              gv *= a.s0[(size_t)w.g * N + n];
              uv *= a.s1[(size_t)w.g * N + n];
            }
            out[orow + n] = f32_to_bf16(silu(gv) * uv);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = w.n0 + wn * 64 + j * 16 + lr;
          if (n < N) {
            float ov = acc[i][j][v];
            if (I8) ov *= a.s0[(size_t)w.g * N + n];
            out[orow + n] = f32_to_bf16(ov);
          }
        }
      }
    }
  }
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

__device__ __forceinline__ void i8x16_to_bf16x16(const uint4& q, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t v = (int32_t)w[i];
    o[2 * i] = pack_bf16x2((float)((v << 24) >> 24), (float)((v << 16) >> 24));
    o[2 * i + 1] = pack_bf16x2((float)((v << 8) >> 24), (float)(v >> 24));
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// ------------------------------------------------------------------------------------------
// general kernel: MODE 0: h = silu(x W_gate^T) * (x W_up^T); MODE 1: rows = h W_down^T
// ------------------------------------------------------------------------------------------
template <int MODE, bool I8>
__global__ __launch_bounds__(THREADS) void k_gemm(const GemmArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  Work w;
  if (!map_work_t<BM>(a, w)) return;
  const int K = a.K;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // A: 128 rows x 8 chunks of 16 B per K-step; thread owns rows tid/8 + 32*i, chunk tid%8
  constexpr int A_LOADS = BM * 8 / THREADS;
  const int a_chunk = tid % 8;
  const uint16_t* a_src[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) a_src[i] = a_row_t<MODE>(a, w, w.m0 + tid / 8 + (THREADS / 8) * i);
  // B: 128 rows; bf16: 8 chunks of 16 B per row, int8: 4 chunks of 16 B per row
  constexpr int B_CPR = I8 ? 4 : 8;
  constexpr int B_LOADS = BN * B_CPR / THREADS;
  const int b_chunk = tid % B_CPR;
  const unsigned char* b_src[B_LOADS];
  int b_rowi[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    b_rowi[i] = tid / B_CPR + (THREADS / B_CPR) * i;
    b_src[i] = b_row_t<MODE, BN>(a, w, b_rowi[i], I8 ? 1 : 2);
  }

  uint4 ra[A_LOADS], rb[B_LOADS];
  auto load_stage = [&](int kt) {
    const int kb = kt * BK;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int col = kb + a_chunk * 8;
      ra[i] = col < K ? *reinterpret_cast<const uint4*>(a_src[i] + col) : zero4();
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int col = kb + b_chunk * (I8 ? 16 : 8);
      const size_t off = (size_t)col * (I8 ? 1 : 2);
      rb[i] = col < K ? *reinterpret_cast<const uint4*>(b_src[i] + off) : zero4();
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* As = lds + buf * STAGE_ELEMS;
    uint16_t* Bs = As + A_ELEMS;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      *reinterpret_cast<uint4*>(As + (tid / 8 + (THREADS / 8) * i) * PITCH + a_chunk * 8) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      uint16_t* dst = Bs + b_rowi[i] * PITCH;
      if (I8) {
        uint4 lo, hi;
        i8x16_to_bf16x16(rb[i], lo, hi);
        *reinterpret_cast<uint4*>(dst + b_chunk * 16) = lo;
        *reinterpret_cast<uint4*>(dst + b_chunk * 16 + 8) = hi;
      } else {
        *reinterpret_cast<uint4*>(dst + b_chunk * 8) = rb[i];
      }
    }
  };

  const int wm = wave / 2, wn = wave % 2;
  const int lr = lane % 16, lk = (lane / 16) * 8;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) brow[j] = b_frag_row<MODE>(wn, j, lr);
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint16_t* As = lds + (kt & 1) * STAGE_ELEMS;
    const uint16_t* Bs = As + A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 16 + lr) * PITCH + ks + lk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + brow[j] * PITCH + ks + lk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage((kt + 1) & 1);
    __syncthreads();
  }
  store_tile<MODE, I8>(a, w, wm, wn, lane, acc);
}

// ------------------------------------------------------------------------------------------
// ring kernel (bf16 weights, K % 32 == 0)
// ------------------------------------------------------------------------------------------
// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));  // vmcnt bits [3:0] and [15:14]
}
// wait until at most `ahead` stages of LPS loads each (0 <= ahead <= MAXA) are still pending
template <int LPS, int MAXA>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (MAXA >= 4) {
    if (ahead >= 4) return wait_vmcnt<4 * LPS>();
  }
  if constexpr (MAXA >= 3) {
    if (ahead == 3) return wait_vmcnt<3 * LPS>();
  }
  if constexpr (MAXA >= 2) {
    if (ahead == 2) return wait_vmcnt<2 * LPS>();
  }
  if (ahead == 1) return wait_vmcnt<LPS>();
  wait_vmcnt<0>();
}

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

// Tile RBM x TBN (gate/up: TBN/2 gate + the same TBN/2 up channels), TBN = 256 or 128; four
// wavefronts side by side, each owning all RBM rows and TBN/4 columns (gate/up: TBN/8 gate +
// the same up channels); K advances RBK=32 per stage through an NST-deep ring (two
// workgroups per CU fit in LDS).
constexpr int RBM = 128, RWN = 4;
constexpr int R_THREADS = 64 * RWN;
constexpr int R_TI = RBM / 16;  // 16-row MFMA slices per tile
constexpr int R_A_BYTES = RBM * RBK * 2;
constexpr int R_DMA_A = RBM / 16 / RWN;  // A loads per stage per wavefront

// Stage geometry for bf16 (W8 = false) or int8 (W8 = true) weights: TBN B rows of RBK weights.
template <bool W8, int TBN>
struct RingB {
  static constexpr int TJ = TBN / RWN / 16;               // 16-column MFMA tiles per wavefront
  static constexpr int ROW = RBK * (W8 ? 1 : 2);          // bytes per B row per stage
  static constexpr int BYTES = TBN * ROW;
  static constexpr int STAGE = R_A_BYTES + BYTES;
  static constexpr int LPR = ROW / 16;                     // DMA lanes per B row
  static constexpr int RPI = 64 / LPR;                     // B rows per DMA load
  static constexpr int DMA = TBN / RPI / RWN;              // B loads per stage per wavefront
  static constexpr int LPS = R_DMA_A + DMA;                // loads per stage per wavefront
  static constexpr int NST = TBN == 128 ? kRing128 : 3;    // stages in the ring
  static constexpr size_t LDS = (size_t)NST * STAGE;
  // waves per SIMD the registers are sized for: 2 with 32 accumulator tiles per wavefront,
  // 3 with 16 when the LDS holds three workgroups per CU (160 KiB)
  static constexpr int WAVES_PER_EU = (TJ == 2 && 160 * 1024 / LDS >= 3) ? 3 : 2;
  static_assert(DMA * RPI * RWN == TBN && TJ % 2 == 0, "tile split");
  static_assert((NST - 2) * LPS < 64 && NST >= 3 && NST <= 6, "vmcnt range");
};

template <int MODE, bool W8, int TBN>
__global__ __launch_bounds__(R_THREADS) __attribute__((amdgpu_waves_per_eu(
    RingB<W8, TBN>::WAVES_PER_EU))) void k_gemm_ring(const GemmArgs a) {
  using B = RingB<W8, TBN>;
  constexpr int R_TJ = B::TJ;
  extern __shared__ __align__(16) unsigned char rlds[];
  Work w;
  if (!map_work_t<RBM>(a, w)) return;
  const int K = a.K;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // DMA assignment: a stage holds RBM A-rows of 64 B, then TBN B-rows of B::ROW bytes (64
  // for bf16, 32 for int8); one 1 KiB load covers 16 A rows or B::RPI B rows.  Wavefront
  // `wave` issues A loads q = wave*R_DMA_A + i and B loads q = wave*B::DMA + i.  Lane l of
  // an A load fills row 16q + l/4, 16-byte position l%4, with the row's chunk
  // (l%4) ^ swz(row), swz(row) = (row >> 2) & 3 (bf16 B rows alike).  Lane l of an int8 B
  // load fills row 32q + l/2, half l%2, with the row's half (l%2) ^ swz8(row),
  // swz8(row) = (row >> 3) & 1.  The swizzles keep the operand reads free of bank conflicts.
  const uint16_t* a_src[R_DMA_A];
  const unsigned char* b_src[B::DMA];
  int ca[R_DMA_A], cb[B::DMA];
#pragma unroll
  for (int i = 0; i < R_DMA_A; ++i) {
    const int row = 16 * (wave * R_DMA_A + i) + lane / 4;
    ca[i] = ((lane % 4) ^ ((row >> 2) & 3)) * 8;
    a_src[i] = a_row_t<MODE>(a, w, w.m0 + row);
  }
#pragma unroll
  for (int i = 0; i < B::DMA; ++i) {
    const int row = B::RPI * (wave * B::DMA + i) + lane / B::LPR;
    cb[i] = W8 ? ((lane % 2) ^ ((row >> 3) & 1)) * 16 : ((lane % 4) ^ ((row >> 2) & 3)) * 16;  // bytes
    b_src[i] = b_row_t<MODE, TBN>(a, w, row, W8 ? 1 : 2);
  }
  auto issue = [&](int kt) {
    unsigned char* st = rlds + (kt % B::NST) * B::STAGE;
    const int kb = kt * RBK;
#pragma unroll
    for (int i = 0; i < R_DMA_A; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(a_src[i] + kb + ca[i]),
                                       (lds_void*)(st + (wave * R_DMA_A + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < B::DMA; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(b_src[i] + kb * (W8 ? 1 : 2) + cb[i]),
                                       (lds_void*)(st + R_A_BYTES + (wave * B::DMA + i) * 1024), 16,
                                       0, 0);
  };

  const int wn = wave, lr = lane % 16;
  // operand reads: row r (a multiple of 16 plus lr), logical chunk c = lane/16 (16 bytes of
  // bf16, or 8 bytes of int8) -> byte offset r*64 + ((c ^ swz(r)) * 16) for bf16,
  // r*32 + (((c >> 1) ^ swz8(r)) * 16) + (c & 1) * 8 for int8
  const int rd_chunk = ((lane / 16) ^ ((lr >> 2) & 3)) * 16;
  int a_off[R_TI], b_off[R_TJ];
#pragma unroll
  for (int i = 0; i < R_TI; ++i) a_off[i] = (i * 16 + lr) * 64 + rd_chunk;
#pragma unroll
  for (int j = 0; j < R_TJ; ++j) {
    int row;
    if (MODE == 0)  // first half of the tiles: gate channels, second half: the same up channels
      row = (j < R_TJ / 2 ? 0 : TBN / 2) + wn * (TBN / RWN / 2) + (j % (R_TJ / 2)) * 16 + lr;
    else
      row = wn * (TBN / RWN) + j * 16 + lr;
    const int c = lane / 16;
    b_off[j] = R_A_BYTES + (W8 ? row * 32 + (((c >> 1) ^ ((row >> 3) & 1)) * 16) + (c & 1) * 8
                               : row * 64 + rd_chunk);
  }
  // 16-row slices of the tile that hold rows of the group; the MFMAs of the others (the
  // padding of a group's last tile) are skipped
  const int ni = min(R_TI, (w.M - w.m0 + 15) / 16);

  // acc[i][j] is the transposed 16x16 product (weights as the first operand), so each lane
  // ends up with 4 consecutive output channels of one row
  f32x4 acc[R_TI][R_TJ];
#pragma unroll
  for (int i = 0; i < R_TI; ++i)
#pragma unroll
    for (int j = 0; j < R_TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / RBK;
#pragma unroll
  for (int s = 0; s < B::NST - 1; ++s)
    if (s < nk) issue(s);
  // the K loop, instantiated per number of live 16-row slices so that it has no branches
  auto k_loop = [&](auto live) {
    constexpr int NI = decltype(live)::value;
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt is complete once at most (stages issued after it) * B::LPS loads are pending
      const int ahead = min(nk - 1, kt + B::NST - 2) - kt;
      wait_ahead<B::LPS, B::NST - 2>(ahead);
      // Every wavefront waited for its own loads of stage kt above, so after this barrier the
      // whole stage is in LDS and every wavefront is done with stage kt-1.  A plain
      // s_barrier: __syncthreads() would add a release fence, i.e. wait for all loads in flight.
      asm volatile("s_barrier" ::: "memory");
      if (kt + B::NST - 1 < nk) issue(kt + B::NST - 1);
      const unsigned char* st = rlds + (kt % B::NST) * B::STAGE;
      bf16x8 bfr[R_TJ], af[NI];
#pragma unroll
      for (int j = 0; j < R_TJ; ++j)
        bfr[j] = W8 ? i8x8_to_bf16x8(*reinterpret_cast<const uint2*>(st + b_off[j]))
                    : *reinterpret_cast<const bf16x8*>(st + b_off[j]);
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = *reinterpret_cast<const bf16x8*>(st + a_off[i]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < R_TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  };
  static_assert(R_TI == 8, "one K-loop instance per live-slice count");
  switch (ni) {
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    case 4: k_loop(std::integral_constant<int, 4>{}); break;
    case 5: k_loop(std::integral_constant<int, 5>{}); break;
    case 6: k_loop(std::integral_constant<int, 6>{}); break;
    case 7: k_loop(std::integral_constant<int, 7>{}); break;
    default: k_loop(std::integral_constant<int, 8>{}); break;
  }

  // epilogue: lane holds output channels 4*(lane/16) + v (v = 0..3) of tile row lane%16;
  // they are written as one 8-byte store per row and tile
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const int N = a.N;
  const int c4 = 4 * (lane / 16);
#pragma unroll
  for (int i = 0; i < R_TI; ++i) {
    const int m = w.m0 + i * 16 + lr;
    if (m >= w.M) continue;
    uint16_t* orow = out + (size_t)(w.r0 + m) * N;
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < R_TJ / 2; ++j) {
        const int n = w.n0 + wn * (TBN / RWN / 2) + j * 16 + c4;  // N % 16 == 0: all 4 or none
        if (n < N) {
          f32x4 g = acc[i][j], u = acc[i][j + R_TJ / 2];
          if (W8) {  // per-channel scales on the fp32 sums
            const float4 sg = *reinterpret_cast<const float4*>(a.s0 + (size_t)w.g * N + n);
            const float4 su = *reinterpret_cast<const float4*>(a.s1 + (size_t)w.g * N + n);
            g = g * f32x4{sg.x, sg.y, sg.z, sg.w};
            u = u * f32x4{su.x, su.y, su.z, su.w};
          }
          *reinterpret_cast<uint2*>(orow + n) =
              make_uint2(pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]),
                         pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < R_TJ; ++j) {
        const int n = w.n0 + wn * (TBN / RWN) + j * 16 + c4;
        if (n < N) {
          f32x4 o = acc[i][j];
          if (W8) {
            const float4 sd = *reinterpret_cast<const float4*>(a.s0 + (size_t)w.g * N + n);
            o = o * f32x4{sd.x, sd.y, sd.z, sd.w};
          }
          *reinterpret_cast<uint2*>(orow + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// ring kernel with 64-deep weight blocks (K % 64 == 0)
// ------------------------------------------------------------------------------------------
// The same tile, wavefront layout, operand order and epilogue as k_gemm_ring, with the LDS
// split into two 8 KiB activation slots (32 K per step) and two weight slots of 64 K per
// block.  A bf16 weight row gives a block 128 bytes, one whole cache line, so one weight DMA
// instruction covers 8 rows x 128 bytes instead of 16 rows x 64 bytes; an int8 row gives 64
// bytes (16 rows per instruction instead of 32 rows x 32 bytes).  Half as many cache lines
// per weight byte, which is what the weight path of the 32-deep ring pays for.  A weight
// block is issued one block (two steps) ahead of its use, an activation step one step ahead.
template <bool W8, int TBN>
struct Ring64 {
  static constexpr int TJ = TBN / RWN / 16;            // 16-column MFMA tiles per wavefront
  static constexpr int A_SLOT = R_A_BYTES;              // 128 rows x 64 bytes
  static constexpr int ROW = W8 ? 64 : 128;             // bytes of a weight row per block
  static constexpr int B_SLOT = TBN * ROW;
  static constexpr int LDS = 2 * A_SLOT + 2 * B_SLOT;   // bf16 80 / 48 KiB, int8 48 / 32 KiB
  static constexpr int LPR = ROW / 16;                  // DMA lanes per weight row
  static constexpr int RPI = 64 / LPR;                  // weight rows per DMA load
  static constexpr int DMA_B = TBN / RPI / RWN;         // weight loads per block per wavefront
  // 3 waves per SIMD only with 16 accumulator tiles per wavefront and room for 3 workgroups
  static constexpr int WAVES_PER_EU = (TJ == 2 && 160 * 1024 / LDS >= 3) ? 3 : 2;
  static_assert(DMA_B * RPI * RWN == TBN && TJ % 2 == 0, "tile split");
  // 16-byte chunk swizzle of weight row r: keeps the 16 rows an operand read touches on
  // distinct banks (8 chunks per bf16 row, 4 per int8 row)
  static __device__ __forceinline__ int swz(int r) { return W8 ? (r >> 2) & 3 : (r >> 1) & 7; }
};

template <int MODE, bool W8, int TBN>
__global__ __launch_bounds__(R_THREADS) __attribute__((amdgpu_waves_per_eu(
    Ring64<W8, TBN>::WAVES_PER_EU))) void k_gemm_ring64(const GemmArgs a) {
  using B = Ring64<W8, TBN>;
  constexpr int R_TJ = B::TJ;
  extern __shared__ __align__(16) unsigned char rlds[];
  Work w;
  if (!map_work_t<RBM>(a, w)) return;
  const int K = a.K;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // Activation DMA as in k_gemm_ring: load q = wave*R_DMA_A + i fills rows 16q .. 16q+15,
  // lane l row 16q + l/4, 16-byte position l%4 with the row's chunk (l%4) ^ ((row >> 2) & 3).
  // Weight DMA: load q = wave*DMA_B + i fills rows RPI*q .. RPI*q + RPI-1, lane l row
  // RPI*q + l/LPR, 16-byte position l%LPR with the row's chunk (l%LPR) ^ swz(row).
  const uint16_t* a_src[R_DMA_A];
  int ca[R_DMA_A];
#pragma unroll
  for (int i = 0; i < R_DMA_A; ++i) {
    const int row = 16 * (wave * R_DMA_A + i) + lane / 4;
    ca[i] = ((lane % 4) ^ ((row >> 2) & 3)) * 8;
    a_src[i] = a_row_t<MODE>(a, w, w.m0 + row);
  }
  const unsigned char* b_src[B::DMA_B];
#pragma unroll
  for (int i = 0; i < B::DMA_B; ++i) {
    const int row = B::RPI * (wave * B::DMA_B + i) + lane / B::LPR;
    b_src[i] = b_row_t<MODE, TBN>(a, w, row, W8 ? 1 : 2) + ((lane % B::LPR) ^ B::swz(row)) * 16;
  }
  auto issue_a = [&](int kt) {  // step kt (32 K) into activation slot kt % 2
    unsigned char* st = rlds + (kt & 1) * B::A_SLOT;
#pragma unroll
    for (int i = 0; i < R_DMA_A; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(a_src[i] + kt * RBK + ca[i]),
                                       (lds_void*)(st + (wave * R_DMA_A + i) * 1024), 16, 0, 0);
  };
  auto issue_b = [&](int jb) {  // block jb (64 K) into weight slot jb % 2
    unsigned char* st = rlds + 2 * B::A_SLOT + (jb & 1) * B::B_SLOT;
#pragma unroll
    for (int i = 0; i < B::DMA_B; ++i)
      __builtin_amdgcn_global_load_lds((global_void*)(b_src[i] + jb * B::ROW),
                                       (lds_void*)(st + (wave * B::DMA_B + i) * 1024), 16, 0, 0);
  };

  const int wn = wave, lr = lane % 16;
  const int rd_chunk = ((lane / 16) ^ ((lr >> 2) & 3)) * 16;
  int a_off[R_TI];
#pragma unroll
  for (int i = 0; i < R_TI; ++i) a_off[i] = (i * 16 + lr) * 64 + rd_chunk;
  // weight operand of tile j in half h of a block: row r, logical chunk c = 4h + lane/16 of
  // the row's 16-byte (bf16) or 8-byte (int8) pieces
  int b_off[2][R_TJ];
#pragma unroll
  for (int j = 0; j < R_TJ; ++j) {
    int row;
    if (MODE == 0)  // first half of the tiles: gate channels, second half: the same up channels
      row = (j < R_TJ / 2 ? 0 : TBN / 2) + wn * (TBN / RWN / 2) + (j % (R_TJ / 2)) * 16 + lr;
    else
      row = wn * (TBN / RWN) + j * 16 + lr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * 4 + lane / 16;
      b_off[h][j] = W8 ? row * B::ROW + ((c >> 1) ^ B::swz(row)) * 16 + (c & 1) * 8
                       : row * B::ROW + (c ^ B::swz(row)) * 16;
    }
  }
  const int ni = min(R_TI, (w.M - w.m0 + 15) / 16);

  f32x4 acc[R_TI][R_TJ];
#pragma unroll
  for (int i = 0; i < R_TI; ++i)
#pragma unroll
    for (int j = 0; j < R_TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nb = K / 64;
  issue_a(0);
  issue_b(0);
  auto k_loop = [&](auto live) {
    constexpr int NI = decltype(live)::value;
    auto step = [&](const unsigned char* as, const unsigned char* bs, int h) {
      bf16x8 bfr[R_TJ], af[NI];
#pragma unroll
      for (int j = 0; j < R_TJ; ++j)
        bfr[j] = W8 ? i8x8_to_bf16x8(*reinterpret_cast<const uint2*>(bs + b_off[h][j]))
                    : *reinterpret_cast<const bf16x8*>(bs + b_off[h][j]);
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = *reinterpret_cast<const bf16x8*>(as + a_off[i]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < R_TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    };
    for (int jb = 0; jb < nb; ++jb) {
      const unsigned char* bs = rlds + 2 * B::A_SLOT + (jb & 1) * B::B_SLOT;
      const bool more = jb + 1 < nb;
      // step 2jb: its activation step and weight block are the last loads issued.  After the
      // barrier every wavefront is done with step 2jb-1, whose activation slot and (for the
      // weights) block jb-1 are refilled next.
      wait_vmcnt<0>();
      asm volatile("s_barrier" ::: "memory");
      issue_a(2 * jb + 1);
      if (more) issue_b(jb + 1);
      step(rlds, bs, 0);
      // step 2jb+1: complete once at most the next block's weight loads are pending
      if (more)
        wait_vmcnt<B::DMA_B>();
      else
        wait_vmcnt<0>();
      asm volatile("s_barrier" ::: "memory");
      if (more) issue_a(2 * jb + 2);
      step(rlds + B::A_SLOT, bs, 1);
    }
  };
  static_assert(R_TI == 8, "one K-loop instance per live-slice count");
  switch (ni) {
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    case 4: k_loop(std::integral_constant<int, 4>{}); break;
    case 5: k_loop(std::integral_constant<int, 5>{}); break;
    case 6: k_loop(std::integral_constant<int, 6>{}); break;
    case 7: k_loop(std::integral_constant<int, 7>{}); break;
    default: k_loop(std::integral_constant<int, 8>{}); break;
  }

  // epilogue: lane holds output channels 4*(lane/16) + v of tile row lane%16
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const int N = a.N;
  const int c4 = 4 * (lane / 16);
#pragma unroll
  for (int i = 0; i < R_TI; ++i) {
    const int m = w.m0 + i * 16 + lr;
    if (m >= w.M) continue;
    uint16_t* orow = out + (size_t)(w.r0 + m) * N;
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < R_TJ / 2; ++j) {
        const int n = w.n0 + wn * (TBN / RWN / 2) + j * 16 + c4;  // N % 16 == 0: all 4 or none
        if (n < N) {
          f32x4 g = acc[i][j], u = acc[i][j + R_TJ / 2];
          if (W8) {  // per-channel scales on the fp32 sums
            const float4 sg = *reinterpret_cast<const float4*>(a.s0 + (size_t)w.g * N + n);
            const float4 su = *reinterpret_cast<const float4*>(a.s1 + (size_t)w.g * N + n);
            g = g * f32x4{sg.x, sg.y, sg.z, sg.w};
            u = u * f32x4{su.x, su.y, su.z, su.w};
          }
          *reinterpret_cast<uint2*>(orow + n) =
              make_uint2(pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]),
                         pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < R_TJ; ++j) {
        const int n = w.n0 + wn * (TBN / RWN) + j * 16 + c4;
        if (n < N) {
          f32x4 o = acc[i][j];
          if (W8) {
            const float4 sd = *reinterpret_cast<const float4*>(a.s0 + (size_t)w.g * N + n);
            o = o * f32x4{sd.x, sd.y, sd.z, sd.w};
          }
          *reinterpret_cast<uint2*>(orow + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
      }
    }
  }
}

// The ring kernel serves bf16 and int8 weights when both K dimensions are multiples of its
// K-step; both launches of a layer must use the same M-tile (it is baked into the launch plan).
bool use_ring(const LayerDims& L) {
  return (L.wdt == MOE_BF16 || L.wdt == MOE_I8) && L.d % RBK == 0 && L.I % RBK == 0;
}

template <int MODE, bool I8, int TBN>
hipError_t run_ring(const GemmArgs& a, int grid, hipStream_t s) {
  if (a.K % 64 == 0) {  // 64-deep weight blocks
    static LdsFlags done64;
    hipError_t e = set_lds(&k_gemm_ring64<MODE, I8, TBN>, Ring64<I8, TBN>::LDS, done64);
    if (e != hipSuccess) return e;
    return launch(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, k_gemm_ring64<MODE, I8, TBN>, grid,
                  R_THREADS, Ring64<I8, TBN>::LDS, s, a);
  }
  using B = RingB<I8, TBN>;
  static LdsFlags done;
  hipError_t e = set_lds(&k_gemm_ring<MODE, I8, TBN>, B::LDS, done);
  if (e != hipSuccess) return e;
  return launch(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, k_gemm_ring<MODE, I8, TBN>, grid,
                R_THREADS, B::LDS, s, a);
}

// tbn: N-tile width of the ring kernel (256 or 128), 0 for the general kernel
template <int MODE, bool I8>
hipError_t run_gemm(GemmArgs a, int max_tiles, int tbn, hipStream_t s) {
  const int width = tbn ? tbn : BN;
  a.n_blk = MODE == 0 ? width / 2 : width;
  const int nt = (a.N + a.n_blk - 1) / a.n_blk;
  // one workgroup per possible (M-tile, N-tile), rounded up to a multiple of the XCD count
  int grid = max_tiles * nt;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (tbn == 256) return run_ring<MODE, I8, 256>(a, grid, s);
  if (tbn == 128) return run_ring<MODE, I8, 128>(a, grid, s);
  static LdsFlags done;
  hipError_t e = set_lds(&k_gemm<MODE, I8>, GEMM_LDS, done);
  if (e != hipSuccess) return e;
  return launch(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, k_gemm<MODE, I8>, grid, THREADS,
                GEMM_LDS, s, a);
}

// Tuned N-tile widths of the ring kernel.  A rule names one layer shape and the token ranges in
// which the 128-wide tile beat the 256-wide one on MI355X, for the gate/up and the down matrix
// separately, measured under the shape's skewed (Zipf) routing and kept only where two sweeps
// agreed by at least 5%.  Every other shape and token count uses 256.  Under skew the big
// groups (shared experts, popular routed experts) dominate a launch; narrower tiles split
// their work over twice the workgroups, at the price of reading each activation tile twice
// as often, which loses once most groups fill several M-tiles.
struct TokenRange {
  int lo, hi;  // inclusive; lo > hi = empty
};
struct TileRule {
  int d, I, E, k, S, wdt;
  TokenRange gate_up[2], down[2];
};
constexpr TileRule kTileRules[] = {
    // DeepSeek-MoE-shaped layer: 64 routed experts of width 1408, top-6, 2 shared, d = 2048
    {2048, 1408, 64, 6, 2, MOE_BF16, {{17, 48}, {1, 0}}, {{64, 128}, {1, 0}}},
    {2048, 1408, 64, 6, 2, MOE_I8, {{25, 32}, {1, 0}}, {{9, 512}, {1, 0}}},
};

// N-tile width of the ring kernel for one matrix (mode 0 gate/up, 1 down) of a layer at T tokens.
int ring_tile_n(const LayerDims& L, int T, int mode) {
  for (const TileRule& r : kTileRules) {
    if (r.d != L.d || r.I != L.I || r.E != L.E || r.k != L.k || r.S != L.S || r.wdt != L.wdt) continue;
    for (const TokenRange& t : mode == 0 ? r.gate_up : r.down)
      if (T >= t.lo && T <= t.hi) return 128;
  }
  return 256;
}

}  // namespace

int gemm_tile_m(const LayerDims& L) { return use_ring(L) ? RBM : BM; }

hipError_t launch_gemm_ffn(const LayerDims& L, int T, const FfnArgs& f, hipStream_t s) {
  const bool ring = use_ring(L);
  const int tm = ring ? RBM : BM;
  const int max_tiles = (int)plan_max_tiles(T, L.k, L.E, L.S);
  // tiles of height tm can never exceed this bound (the plan is sized for height 16)
  const int tiles = (T * L.k) / tm + (T * L.k < L.E ? T * L.k : L.E) + L.S * ((T + tm - 1) / tm) + 1;
  const int grid_tiles = tiles < max_tiles ? tiles : max_tiles;
  GemmArgs a{};
  a.offsets = f.offsets;
  a.perm = f.perm;
  a.plan = f.plan;
  a.k = L.k;
  a.E = L.E;
  a.max_groups = L.E + L.S;
  const bool i8 = L.wdt == MOE_I8;
  hipError_t err;

  a.in = f.x;
  a.w0 = f.w_gate;
  a.w1 = f.w_up;
  a.s0 = f.s_gate;
  a.s1 = f.s_up;
  a.out = f.h;
  a.K = L.d;
  a.N = L.I;
  int tbn = ring ? ring_tile_n(L, T, 0) : 0;
  err = i8 ? run_gemm<0, true>(a, grid_tiles, tbn, s) : run_gemm<0, false>(a, grid_tiles, tbn, s);
  if (err != hipSuccess) return err;

  a.in = f.h;
  a.w0 = f.w_down;
  a.w1 = nullptr;
  a.s0 = f.s_down;
  a.s1 = nullptr;
  a.out = f.rows;
  a.K = L.I;
  a.N = L.d;
  tbn = ring ? ring_tile_n(L, T, 1) : 0;
  return i8 ? run_gemm<1, true>(a, grid_tiles, tbn, s) : run_gemm<1, false>(a, grid_tiles, tbn, s);
}

}  // namespace moe
