// Grouped GEMM on the bf16 matrix cores for prefill sizes: every expert in one launch.
//
// The switchyard page runs all experts' GEMMs in one launch with the SwiGLU fused into the
// epilogue (§02 "One launch for all experts"); here that is one launch per matrix pair on
// gfx950's v_mfma_f32_16x16x32_bf16.  Work items come from the launch plan written by the
// permute kernel: blockIdx.y is an M-tile (group, first row) of the sorted rows, blockIdx.x
// an N-tile; tiles past the plan's count exit at once, so the grid can be sized from T*k
// without reading counts back to the host.
//
// Tile: BM=128 rows x 128 columns, BK=64, four wavefronts in a 2x2 layout, each owning a
// 64x64 accumulator block (sixteen 16x16 MFMA tiles).  For gate/up the 128 columns are 64
// gate channels followed by the same 64 up channels, and every wavefront holds matching
// gate and up tiles, so silu(g)*u is formed in registers.  A rows are gathered through perm
// (token rows of x) or read in order (h rows); both operands are staged K-contiguous in LDS
// (row pitch padded by 16 bytes), double-buffered with a register prefetch of the next
// K-step.  int8 weights are widened to bf16 (exact) as they are written to LDS; the
// per-channel scale multiplies the fp32 accumulator in the epilogue.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int PITCH = BK + 8;                  // bf16 elements per LDS row
constexpr int A_ELEMS = BM * PITCH, B_ELEMS = BN * PITCH;
constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
constexpr size_t GEMM_LDS = 2 * STAGE_ELEMS * sizeof(uint16_t);

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
};

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

// MODE 0: h = silu(x W_gate^T) * (x W_up^T); MODE 1: rows = h W_down^T
template <int MODE, bool I8>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tile = blockIdx.y;
  const int32_t* plan = a.plan;
  if (tile >= plan[1]) return;
  const int32_t* tiles = plan + kPlanHeader + a.max_groups;
  const int g = tiles[2 * tile], m0 = tiles[2 * tile + 1];
  const int r0 = a.offsets[g];
  const int M = a.offsets[g + 1] - r0;
  const int K = a.K, N = a.N;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // ---- global -> register staging assignments
  // A: 128 rows x 8 chunks of 16 B; thread owns rows (tid/8) + 32*i, chunk tid%8
  const int a_chunk = tid % 8;
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + tid / 8 + 32 * i, M - 1);
    const int r = r0 + m;
    size_t src_row;
    if (MODE == 0)
      src_row = (g < a.E) ? (size_t)(a.perm[r] / a.k) : (size_t)m;
    else
      src_row = (size_t)r;
    a_src[i] = reinterpret_cast<const uint16_t*>(a.in) + src_row * K;
  }
  // B: 128 rows; bf16: 8 chunks of 16 B per row, rows (tid/8) + 32*i
  //              int8: 4 chunks of 16 B per row, rows (tid/4) + 64*i
  constexpr int B_LOADS = I8 ? 2 : 4;
  constexpr int B_CPR = I8 ? 4 : 8;   // 16-byte chunks per row per K-step
  const int b_chunk = tid % B_CPR;
  const unsigned char* b_src[B_LOADS];
  int b_row[B_LOADS];
  const int n_blk = MODE == 0 ? BN / 2 : BN;
  const int n0 = blockIdx.x * n_blk;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int row = tid / B_CPR + (256 / B_CPR) * i;
    b_row[i] = row;
    int n;
    const void* base;
    if (MODE == 0) {
      n = n0 + (row % (BN / 2));
      base = row < BN / 2 ? a.w0 : a.w1;
    } else {
      n = n0 + row;
      base = a.w0;
    }
    n = min(n, N - 1);
    const size_t esz = I8 ? 1 : 2;
    b_src[i] = reinterpret_cast<const unsigned char*>(base) + ((size_t)g * N + n) * K * esz;
  }

  uint4 ra[4], rb[B_LOADS];
  auto load_stage = [&](int kt) {
    const int kb = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(As + (tid / 8 + 32 * i) * PITCH + a_chunk * 8) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      uint16_t* dst = Bs + b_row[i] * PITCH;
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

  // ---- MFMA layout: wave (wm, wn) owns rows wm*64.., 4x4 tiles of 16x16
  const int wm = wave / 2, wn = wave % 2;
  const int lr = lane % 16, lk = (lane / 16) * 8;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (MODE == 0)  // j = 0,1: gate channels; j = 2,3: the same up channels
      brow[j] = (j < 2 ? 0 : BN / 2) + wn * 32 + (j % 2) * 16 + lr;
    else
      brow[j] = wn * 64 + j * 16 + lr;
  }
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

  // ---- epilogue: lane holds rows 4*(lane/16) + v, column lane%16 of each 16x16 tile
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * 64 + i * 16 + (lane / 16) * 4 + v;
      if (m >= M) continue;
      const size_t orow = (size_t)(r0 + m) * N;
      if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 32 + j * 16 + lr;
          if (n < N) {
            float gv = acc[i][j][v], uv = acc[i][j + 2][v];
            if (I8) {
              gv *= a.s0[(size_t)g * N + n];
              uv *= a.s1[(size_t)g * N + n];
            }
            out[orow + n] = f32_to_bf16(silu(gv) * uv);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + lr;
          if (n < N) {
            float ov = acc[i][j][v];
            if (I8) ov *= a.s0[(size_t)g * N + n];
            out[orow + n] = f32_to_bf16(ov);
          }
        }
      }
    }
  }
}

template <int MODE, bool I8>
hipError_t run_gemm(const GemmArgs& a, int max_tiles, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<MODE, I8>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_blk = MODE == 0 ? BN / 2 : BN;
  dim3 grid((a.N + n_blk - 1) / n_blk, max_tiles);
  LaunchTimer timer(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, s);
  k_gemm<MODE, I8><<<grid, 256, GEMM_LDS, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_m() { return BM; }

hipError_t launch_gemm_ffn(const LayerDims& L, int T, const FfnArgs& f, hipStream_t s) {
  const int max_tiles = (int)plan_max_tiles(T, L.k, L.E, L.S);
  // tiles of height BM can never exceed this bound (it is computed for height 16)
  const int tiles = (T * L.k) / BM + (T * L.k < L.E ? T * L.k : L.E) + L.S * ((T + BM - 1) / BM) + 1;
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
  err = i8 ? run_gemm<0, true>(a, grid_tiles, s) : run_gemm<0, false>(a, grid_tiles, s);
  if (err != hipSuccess) return err;

  a.in = f.h;
  a.w0 = f.w_down;
  a.w1 = nullptr;
  a.s0 = f.s_down;
  a.s1 = nullptr;
  a.out = f.rows;
  a.K = L.I;
  a.N = L.d;
  return i8 ? run_gemm<1, true>(a, grid_tiles, s) : run_gemm<1, false>(a, grid_tiles, s);
}

}  // namespace moe
