// Grouped GEMV for decode sizes: every touched expert in one launch, weights streamed once.
//
// At decode sizes an expert sees one to a few rows, so the layer is bound by reading the
// touched experts' weights from HBM (the switchyard page's decode path is a grouped GEMV that
// streams the expert weights, §02 "One launch for all experts").  What decides the speed is
// how many bytes each CU keeps in flight, so the kernel is built around that:
//
//  * blockIdx.y walks the touched groups of the launch plan, blockIdx.x a block of NB
//    output channels of that group's weight matrix (or matrices: gate and up together);
//    consecutive blocks stream consecutive stretches of one matrix;
//  * the K dimension is split across the block's four wavefronts; inside a wavefront,
//    eight lanes own one channel and read its weight row in 128-byte coalesced runs;
//  * every weight load of the block is issued at once into registers before any math
//    (about 16 x 16 B per lane), so a block costs about one memory round trip and several
//    blocks per CU overlap theirs; the weights then stay in registers while the group's
//    activation rows are processed in chunks of up to MB rows staged in LDS, by
//    direct-to-LDS loads issued right behind the weights so that both round trips overlap;
//  * partial sums are reduced over the 8 lanes with DPP moves and over the 4 wavefronts
//    through LDS in a fixed order, so results are bit-reproducible;
//  * the epilogue applies the int8 per-channel scale, the SwiGLU (gate/up) and the
//    rounding to the activation type.
//
// A second kernel, k_gemv_mfma, keeps this structure and does the math on the matrix cores,
// for groups of a few dozen rows (described at its definition).
//
// Weight x activation types: f32 x f32 (fp32 FMA), bf16 x bf16 (v_dot2_f32_bf16), int8 x bf16
// (int8 -> bf16 is exact for |q| <= 127, then v_dot2_f32_bf16; the scale multiplies the fp32
// sum once per channel).
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
  int K, N, k, E;
  int mb_max;       // rows staged per chunk (<= the kernel's MB)
};

constexpr int kWaves = 4;

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gmem_void;
// read-only for the kernel's lifetime (the sort wrote it in an earlier launch): through the
// constant address space a wave-uniform lookup becomes a scalar load even after the kernel's
// own stores, so it does not wait behind the vector loads in flight
typedef const __attribute__((address_space(4))) int32_t cint32;
// s_waitcnt immediates: only lgkmcnt = 0 (vmcnt and expcnt left at their maxima), only vmcnt = 0
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int kWaitVm0 = 0x0F70;

template <typename WT> struct WTraits;
template <> struct WTraits<float> { static constexpr int V = 4; };  // weights per 16-byte load
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
// CPG: channels per 8-lane group (NB = 8 * CPG channels per block);
// MAXIT: K steps (8 lanes x 16 B) per wavefront per round;
// MB: rows per chunk (a group with more rows takes further chunks: with one round over K the
// weights stay in registers, so a small MB costs no traffic and saves accumulator registers).
// grid: (ceil(N / NB), slots); block 256; dynamic LDS mb_max * ROUND * sizeof(AT).
// blockIdx.x is dispatched fastest, so the blocks in flight read consecutive N-blocks of
// one expert: one contiguous stretch of memory streamed in order (measured 25% faster
// than spreading the blocks in flight over many experts at the same offset).
template <int MODE, typename AT, typename WT, int CPG, int MAXIT, int MB>
__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a) {
  constexpr int NMAT = MODE == 0 ? 2 : 1;
  constexpr int NB = 8 * CPG;
  constexpr int V = WTraits<WT>::V;             // weights per 16-byte load
  constexpr int STEP = 8 * V;                   // K elements per 8-lane step
  constexpr int ROUND = kWaves * MAXIT * STEP;  // K elements per round
  typedef Dot<AT, WT> D;
  extern __shared__ __align__(16) unsigned char xs[];
  __shared__ float red[kWaves][CPG][NMAT][MB][8];

  const int slot = blockIdx.y;
  if (slot >= a.plan[0]) return;
  const int g = a.plan[kPlanHeader + slot];
  const int K = a.K, N = a.N;
  const int n0 = blockIdx.x * NB;
  const int r0 = a.offsets[g];
  const int Mg = a.offsets[g + 1] - r0;
  const int M = (g < a.E && a.plan[3] > 0) ? min(Mg, a.plan[3]) : Mg;  // capacity: the rest is dropped

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int q = lane % 8, lg = lane / 8;
  const AT* in = reinterpret_cast<const AT*>(a.in);
  const int rounds = (K + ROUND - 1) / ROUND;
  const int row_bytes = ROUND * (int)sizeof(AT);

  // weight rows of this lane's channels (clamped into the matrix; results discarded)
  const WT* wp[CPG][NMAT];
#pragma unroll
  for (int c = 0; c < CPG; ++c) {
    const size_t row = ((size_t)g * N + min(n0 + c * 8 + lg, N - 1)) * K;
    wp[c][0] = reinterpret_cast<const WT*>(a.w0) + row;
    if (NMAT == 2) wp[c][NMAT - 1] = reinterpret_cast<const WT*>(a.w1) + row;
  }

  uint4 wbuf[CPG][NMAT][MAXIT];
  float acc[CPG][NMAT][MB];
  for (int m0 = 0; m0 < M; m0 += a.mb_max) {
    const int mb = min(a.mb_max, M - m0);
#pragma unroll
    for (int c = 0; c < CPG; ++c)
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[c][t][m] = 0.f;

    for (int rd = 0; rd < rounds; ++rd) {
      const int k_round = rd * ROUND;
      const int cols = min(ROUND, K - k_round);
      const int steps = (cols + STEP - 1) / STEP;  // 8-lane steps in this round
      const int spw = (steps + kWaves - 1) / kWaves;
      const int s_lo = wave * spw, s_hi = min(steps, s_lo + spw);
      // (1) weights -> registers, all loads in flight at once (kept for every row chunk
      //     when one round covers K)
      if (m0 == 0 || rounds > 1) {
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
          const int col = k_round + (s_lo + it) * STEP + q * V;
          const bool ok = (s_lo + it < s_hi) && col < K;
#pragma unroll
          for (int c = 0; c < CPG; ++c)
#pragma unroll
            for (int t = 0; t < NMAT; ++t)
              wbuf[c][t][it] = ok ? *reinterpret_cast<const uint4*>(wp[c][t] + col) : make_uint4(0, 0, 0, 0);
        }
      }
      // (2) activation rows m0 .. m0+mb-1, columns of this round -> LDS by direct-to-LDS
      //     loads (one instruction moves 64 chunks of 16 bytes of one row; no registers),
      //     issued right behind the weights.  The row lookups are wave-uniform scalar loads,
      //     so nothing here waits for the weights: the barrier that keeps the previous row
      //     chunk's LDS reads ahead of the new rows needs only those reads (lgkmcnt), not the
      //     loads in flight, which __syncthreads() would wait for.
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      asm volatile("s_barrier" ::: "memory");
      const int chunks = cols * (int)sizeof(AT) / 16;  // per row
      const int ipr = (chunks + kWave - 1) / kWave;     // instructions per row
      // wave index made visibly uniform, so the lookups below become scalar loads
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      for (int j = wave_u; j < mb * ipr; j += kWaves) {
        const int m = j / ipr, c0 = (j % ipr) * kWave;
        const int r = r0 + m0 + m;
        size_t src_row;
        if (MODE == 0)
          src_row = (g < a.E) ? (size_t)(((const cint32*)a.perm)[r] / a.k) : (size_t)(m0 + m);
        else
          src_row = (size_t)r;
        const int cc = c0 + lane;
        if (cc < chunks)  // lane cc's 16 bytes land at the instruction's LDS base + 16 * lane
          __builtin_amdgcn_global_load_lds(
              (gmem_void*)(in + src_row * K + k_round + cc * (16 / (int)sizeof(AT))),
              (lds_void*)(xs + m * row_bytes + c0 * 16), 16, 0, 0);
      }
      // this wavefront's weights and rows are in; the barrier makes every wavefront's rows visible
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      asm volatile("s_barrier" ::: "memory");
      // (3) math
#pragma unroll
      for (int it = 0; it < MAXIT; ++it) {
        const int st = s_lo + it;
        const int xcol = st * STEP + q * V;  // column within the round
        if (st < s_hi && xcol < cols) {
          const unsigned char* xp = xs + xcol * (int)sizeof(AT);
#pragma unroll
          for (int c = 0; c < CPG; ++c)
#pragma unroll
            for (int t = 0; t < NMAT; ++t) {
              const typename D::W w = D::prep(wbuf[c][t][it]);
#pragma unroll
              for (int m = 0; m < MB; ++m)
                if (m < mb) acc[c][t][m] = D::run(w, xp + m * row_bytes, acc[c][t][m]);
            }
        }
      }
    }
    // (4) reduce over the 8 lanes of each channel (DPP), then over the wavefronts (LDS,
    //     fixed order), then the epilogue
#pragma unroll
    for (int c = 0; c < CPG; ++c)
#pragma unroll
      for (int t = 0; t < NMAT; ++t)
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float v = sum8(settle_dot(acc[c][t][m]));
          if (m == q) red[wave][c][t][m][lg] = v;
        }
    __syncthreads();
    if (wave == 0 && q < mb) {
      const int m = q;
      const size_t orow = (size_t)(r0 + m0 + m) * N;
#pragma unroll
      for (int c = 0; c < CPG; ++c) {
        const int n = n0 + c * 8 + lg;
        if (n < N) {
          float v[NMAT];
#pragma unroll
          for (int t = 0; t < NMAT; ++t)
            v[t] = (red[0][c][t][m][lg] + red[1][c][t][m][lg]) + (red[2][c][t][m][lg] + red[3][c][t][m][lg]);
          if (MODE == 0) {
            float gv = v[0], uv = v[NMAT - 1];
            if (a.s0) {
              gv *= a.s0[(size_t)g * N + n];
              uv *= a.s1[(size_t)g * N + n];
            }
            Act<AT>::store(reinterpret_cast<AT*>(a.out), orow + n, silu(gv) * uv);
          } else {
            float ov = v[0];
            if (a.s0) ov *= a.s0[(size_t)g * N + n];
            Act<AT>::store(reinterpret_cast<AT*>(a.out), orow + n, ov);
          }
        }
      }
    }
  }
}

template <int MODE, typename AT, typename WT, int CPG, int MAXIT, int MB>
hipError_t run_gemv(GemvArgs a, int T, int slots, hipStream_t s) {
  constexpr int V = WTraits<WT>::V;
  constexpr int ROUND = kWaves * MAXIT * 8 * V;
  a.mb_max = T < MB ? T : MB;  // no group holds more than T rows
  dim3 grid((a.N + 8 * CPG - 1) / (8 * CPG), slots);
  const size_t lds = (size_t)a.mb_max * ROUND * sizeof(AT);
  return launch(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, k_gemv<MODE, AT, WT, CPG, MAXIT, MB>,
                grid, 256, lds, s, a);
}

// Pick MAXIT (K steps per wavefront) so one round covers K when possible, and CPG (channel
// groups per block).  Measured on the OLMoE and DeepSeek shapes: more, smaller blocks beat
// fewer blocks with more loads per lane once a block's loads fill a round trip, so the down
// projection and int8 gate/up (a lane's 16 bytes hold twice the weights) use 1 channel
// group when a wavefront covers K in 4-8 steps (down at CPG 1 against 2: -4% at OLMoE T=8,
// -8% at DeepSeek T=8).  Rows
// go in chunks of 4 when one round covers K (the registers saved raise the occupancy the
// bandwidth follows; at T = 1 and 2 chunks of T, 2-4% faster still; gate/up past T=4 in
// chunks of 8), else of 8 (each further chunk would read the weights again).
template <int MODE, typename AT, typename WT>
hipError_t dispatch_gemv(const GemvArgs& a, int T, int slots, hipStream_t s) {
  constexpr int V = WTraits<WT>::V;
  constexpr int NMAT = MODE == 0 ? 2 : 1;
  const int steps = (a.K + 8 * V - 1) / (8 * V);
  const int spw = (steps + kWaves - 1) / kWaves;
  if (spw <= 2) return run_gemv<MODE, AT, WT, (NMAT == 2 ? 4 : 2), 2, 4>(a, T, slots, s);
  if (spw <= 4) {
    constexpr int C = NMAT == 1 || V == 16 ? 1 : 2;
    if (T == 1) return run_gemv<MODE, AT, WT, C, 4, 1>(a, T, slots, s);
    if (T == 2) return run_gemv<MODE, AT, WT, C, 4, 2>(a, T, slots, s);
    return run_gemv<MODE, AT, WT, C, 4, 4>(a, T, slots, s);
  }
  if (spw <= 8) {
    if (T == 1) return run_gemv<MODE, AT, WT, 1, 8, 1>(a, T, slots, s);
    if (T == 2) return run_gemv<MODE, AT, WT, 1, 8, 2>(a, T, slots, s);
    if (T <= 4) return run_gemv<MODE, AT, WT, 1, 8, 4>(a, T, slots, s);
    // gate/up past 4 tokens: chunks of 8 rows (a shared expert's T rows in one pass; DeepSeek
    // T=6/8 gate/up 3-4% faster, OLMoE unchanged); the down projection keeps 4 (8 cost it
    // 9% at DeepSeek T=8: the extra accumulators lower the occupancy)
    return run_gemv<MODE, AT, WT, 1, 8, (MODE == 0 ? 8 : 4)>(a, T, slots, s);
  }
  return run_gemv<MODE, AT, WT, (NMAT == 2 ? 1 : 2), 8, 8>(a, T, slots, s);
}


// ---------------------------------------------------------------------------------------
// Matrix-core GEMV: the same block shape and weight streaming, for groups of a few to a few
// dozen rows, where the VALU dot products above would cost more than the weights take to
// arrive.  Lanes load weights straight into the operand layout of v_mfma_f32_16x16x32_bf16:
// lane l owns weight row l % 16 of a 16-row tile and, in every 64-K block, the 16 K elements
// 16 * (l / 16) .. +15 (bf16: 32 bytes, so the four lanes of a row read its 128-byte run;
// int8: 16 bytes).  The first MFMA of a block takes elements 0..7 of every lane, the second
// 8..15; the activation operand (token l % 16, the same K elements) is loaded from the
// L2-resident rows in the same pattern, so each MFMA sums 32 matching products.  The K blocks
// are split over the four wavefronts; all of a wavefront's weight loads are issued before any
// math, as in the VALU GEMV, and stay in registers while the group's rows pass in chunks of 16
// tokens.  Partial tiles are summed over the wavefronts through LDS in a fixed order.
// MODE 0: tile j holds gate channels n0+8j .. +7 in rows 0-7 and the same up channels in rows
// 8-15 (NC = 8 * NTI channels per block); MODE 1: tile j holds channels n0+16j .. +15.
// MAXB: 64-K blocks per wavefront per round (a round covers K when K <= 256 * MAXB).
// grid: (ceil(N / NC), slots); block 256; K % 64 == 0; bf16 activations.
template <int MODE, bool W8, int NTI, int MAXB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemv_mfma(const GemvArgs a) {
  constexpr int NC = MODE == 0 ? 8 * NTI : 16 * NTI;
  constexpr int WL = W8 ? 1 : 2;  // 16-byte weight loads per lane per 64-K block
  constexpr int ESZ = W8 ? 1 : 2;
  constexpr int RB = kWaves * MAXB;
  __shared__ f32x4 red[kWaves][NTI][kWave];

  const cint32* plan = (const cint32*)a.plan;
  const int slot = blockIdx.y;
  if (slot >= plan[0]) return;
  const int g = plan[kPlanHeader + slot];
  const int K = a.K, N = a.N;
  const int n0 = blockIdx.x * NC;
  const int r0 = ((const cint32*)a.offsets)[g];
  const int Mg = ((const cint32*)a.offsets)[g + 1] - r0;
  const int M = (g < a.E && plan[3] > 0) ? min(Mg, plan[3]) : Mg;  // capacity: the rest is dropped

  // the wavefront index made visibly uniform, so the K split below is scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int lr = lane % 16, kq = lane / 16;
  const int nbk = K / 64;
  const int rounds = (nbk + RB - 1) / RB;

  // weight row of this lane in each tile (clamped into the matrix; results discarded)
  const unsigned char* wrow[NTI];
#pragma unroll
  for (int j = 0; j < NTI; ++j) {
    const int mat = MODE == 0 ? lr / 8 : 0;
    const int ch = MODE == 0 ? n0 + 8 * j + lr % 8 : n0 + 16 * j + lr;
    const unsigned char* base = reinterpret_cast<const unsigned char*>(mat ? a.w1 : a.w0);
    wrow[j] = base + ((size_t)g * N + min(ch, N - 1)) * (size_t)K * ESZ + kq * 16 * ESZ;
  }
  const uint16_t* in = reinterpret_cast<const uint16_t*>(a.in);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  uint4 wv[NTI][MAXB][WL];
  for (int m0 = 0; m0 < M; m0 += 16) {
    f32x4 acc[NTI];
#pragma unroll
    for (int j = 0; j < NTI; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int rd = 0; rd < rounds; ++rd) {
      const int nb_r = min(RB, nbk - rd * RB);
      const int bpw = (nb_r + kWaves - 1) / kWaves;
      const int b_lo = wave * bpw, b_hi = min(nb_r, b_lo + bpw);
      // blocks past this wavefront's share load the round's last block again (no branches
      // around the loads; their products are skipped)
      const int kb0 = rd * RB + b_lo, kb_last = rd * RB + nb_r - 1;
      if (m0 == 0 || rounds > 1) {
#pragma unroll
        for (int it = 0; it < MAXB; ++it) {
          const size_t off = (size_t)min(kb0 + it, kb_last) * 64 * ESZ;
#pragma unroll
          for (int j = 0; j < NTI; ++j)
#pragma unroll
            for (int u = 0; u < WL; ++u) wv[j][it][u] = *reinterpret_cast<const uint4*>(wrow[j] + off + 16 * u);
        }
      }
      // this lane's token: column lr of the chunk (padding columns repeat the last row)
      const int m = min(m0 + lr, M - 1);
      int src;
      if (MODE == 0) {
        if (g < a.E) {  // 16 wave-uniform (scalar) perm lookups, one picked per lane
          int pv = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int v = ((const cint32*)a.perm)[r0 + min(m0 + i, M - 1)];
            pv = lr == i ? v : pv;
          }
          src = pv / a.k;
        } else {
          src = m;  // a shared expert's rows are the tokens in order
        }
      } else {
        src = r0 + m;
      }
      const unsigned char* xrow = reinterpret_cast<const unsigned char*>(in + (size_t)src * K) + kq * 32;
      uint4 xv[MAXB][2];
#pragma unroll
      for (int it = 0; it < MAXB; ++it) {
        const size_t off = (size_t)min(kb0 + it, kb_last) * 128;
        xv[it][0] = *reinterpret_cast<const uint4*>(xrow + off);
        xv[it][1] = *reinterpret_cast<const uint4*>(xrow + off + 16);
      }
#pragma unroll
      for (int it = 0; it < MAXB; ++it) {
        if (b_lo + it < b_hi) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bf16x8 xb = __builtin_bit_cast(bf16x8, xv[it][h]);
#pragma unroll
            for (int j = 0; j < NTI; ++j) {
              const uint4 q = wv[j][it][W8 ? 0 : h];
              const bf16x8 wb = W8 ? i8x8_to_bf16x8(h == 0 ? make_uint2(q.x, q.y) : make_uint2(q.z, q.w))
                                   : __builtin_bit_cast(bf16x8, q);
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, acc[j], 0, 0, 0);
            }
          }
        }
      }
    }
    // lane l of a tile holds rows 4 * (l / 16) + v (v = 0..3) for token l % 16
#pragma unroll
    for (int j = 0; j < NTI; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    const int mb = min(16, M - m0);
    for (int t = threadIdx.x; t < 16 * NC; t += 256) {
      const int c = t / NC, chl = t % NC;  // token, channel within the block
      const int n = n0 + chl;
      if (c < mb && n < N) {
        const size_t o = (size_t)(r0 + m0 + c) * N + n;
        if (MODE == 0) {
          const int j = chl / 8, i = chl % 8, v = i % 4;
          const int lg = 16 * (i / 4) + c, lu = lg + 32;  // tile rows i and i + 8
          float gv = (red[0][j][lg][v] + red[1][j][lg][v]) + (red[2][j][lg][v] + red[3][j][lg][v]);
          float uv = (red[0][j][lu][v] + red[1][j][lu][v]) + (red[2][j][lu][v] + red[3][j][lu][v]);
          if (a.s0) {
            gv *= a.s0[(size_t)g * N + n];
            uv *= a.s1[(size_t)g * N + n];
          }
          Act<uint16_t>::store(out, o, silu(gv) * uv);
        } else {
          const int j = chl / 16, i = chl % 16, v = i % 4;
          const int l = 16 * (i / 4) + c;
          float ov = (red[0][j][l][v] + red[1][j][l][v]) + (red[2][j][l][v] + red[3][j][l][v]);
          if (a.s0) ov *= a.s0[(size_t)g * N + n];
          Act<uint16_t>::store(out, o, ov);
        }
      }
    }
    __syncthreads();  // the next chunk rewrites red
  }
}

template <int MODE, bool W8, int NTI, int MAXB>
hipError_t run_gemv_mfma(const GemvArgs& a, int slots, hipStream_t s) {
  constexpr int NC = MODE == 0 ? 8 * NTI : 16 * NTI;
  dim3 grid((a.N + NC - 1) / NC, slots);
  return launch(MODE == 0 ? MOE_KERNEL_GATE_UP : MOE_KERNEL_DOWN, k_gemv_mfma<MODE, W8, NTI, MAXB>, grid, 256,
                0, s, a);
}

// Two tiles per block (gate/up: 16 channels of both matrices; down: 32 channels): faster
// than one on the OLMoE and DeepSeek shapes (gate/up at OLMoE T=48 94 against 98 us, down
// 49 against 51 us), the block's 64-128 KiB of weights about one round trip.  MAXB: the
// smallest that covers K in one round (K = 1408 splits 6/6/6/4).
template <int MODE, bool W8>
hipError_t dispatch_gemv_mfma(const GemvArgs& a, int slots, hipStream_t s) {
  const int nbk = a.K / 64;
  if (nbk <= 8) return run_gemv_mfma<MODE, W8, 2, 2>(a, slots, s);
  if (nbk <= 16) return run_gemv_mfma<MODE, W8, 2, 4>(a, slots, s);
  if (nbk <= 24) return run_gemv_mfma<MODE, W8, 2, 6>(a, slots, s);
  return run_gemv_mfma<MODE, W8, 2, 8>(a, slots, s);
}


// ---------------------------------------------------------------------------------------
// Down projection and combine in one launch, for decode sizes inside moe_forward.
//
// The combine needs every row routed to an output channel, so a block here owns 8 output
// channels across all of the launch's touched groups (where k_gemv's block owns them for one
// group): it walks the group list, streams each group's 8 weight rows (one contiguous 8 x K
// stretch), keeps the rows' partial sums in LDS and, at the end, sums each token's rows for
// its channels and writes y.  No block waits for another and the rows never leave LDS, which
// saves the combine's launch and its round trip through memory.
//
//  * Lane layout and arithmetic are k_gemv's (MODE 1): K split over the four wavefronts in
//    spw 8-lane steps each, eight lanes per channel, the same dot-product order, the DPP sum
//    over the 8 lanes, the fixed-order sum over wavefronts, the int8 scale and the rounding
//    to the activation type; the sum over a token's rows then follows k_combine's order with
//    its single rounding.  y is therefore bit-identical to the two launches.
//  * The workgroup is NG slot streams of four wavefronts; stream g takes groups g, g + NG, ...
//    so several groups' weights are in flight per CU.  The wavefronts of one K-slice first
//    stage that slice of all R activation rows into LDS by direct-to-LDS loads, and one
//    barrier, behind the first groups' weight loads, makes the rows visible before the first
//    sum; the next barrier is the one before the combine.
//  * Each stream's weights pass through registers in a ring of D groups: while one group's
//    rows are summed, the next D-1 groups' loads are in flight.  Every weight load is
//    unconditional (a lane past its columns reads an in-bounds piece and skips the math), so
//    the number of loads in flight is a compile-time constant and the compiler's waits leave
//    the ring running; the ring's tail re-reads the last group D times (a cache hit).
// grid: ceil(N / 8); block 256 * NG; one pass covers K (MAXIT == spw); dynamic LDS from
// down_combine_geom().
struct DownCombineArgs {
  const void* h;            // [R, K] gate/up output by sorted row
  const void* w;            // [G, N, K] down weights
  const float* s;           // int8 per-channel scales [G, N], else null
  const int32_t* offsets;
  const int32_t* plan;
  const int32_t* inv_perm;  // [T * k], -1 for a dropped slot
  const float* topk_w;      // [T * k]
  const void* residual;     // [T, N] or null
  void* y;                  // [T, N]
  int T, k, S, E, K, N;
  int R;                    // rows: T * k + S * T
  int slice;                // LDS bytes of one row's wavefront slice: spw * 8 * V * sizeof(AT)
};

constexpr int kDcRing = 2;  // groups in each stream's weight ring (deeper rings measured slower)
// Slot streams per workgroup (four wavefronts each): more streams keep more groups' weights in
// flight per CU.  Measured against one, two and four: two for bf16 weights (OLMoE T=8 layer
// 108-110 against 109-111 us with four), four for int8, whose groups carry half the bytes for
// the same fixed cost per group (T=8 65 against 68 us).
template <typename WT>
constexpr int dc_streams() { return sizeof(WT) == 1 ? 4 : 2; }
constexpr size_t kDcMaxLds = 160 * 1024;  // one workgroup per CU

template <typename AT, typename WT, int MAXIT, int MB, int NG>
__global__ __launch_bounds__(256 * NG) void k_down_combine(const DownCombineArgs a) {
  constexpr int V = WTraits<WT>::V;
  constexpr int STEP = 8 * V;
  constexpr bool I8 = sizeof(WT) == 1;
  constexpr int D = kDcRing;
  typedef Dot<AT, WT> Dt;
  extern __shared__ __align__(16) unsigned char lds[];

  const int R = a.R, K = a.K, N = a.N, T = a.T, k = a.k, Tk = T * k;
  const int tid = threadIdx.x;
  // the wavefront index made visibly uniform: the group lookups below stay scalar loads, and
  // the ring's loop stays a uniform loop (as a divergent one, every lookup became a vector
  // load whose wait drained the ring)
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int kw = wave % kWaves, grp = wave / kWaves;  // K-slice, and the slot stream
  const int q = lane % 8, lg = lane / 8;
  const int n0 = blockIdx.x * 8;
  const int n = min(n0 + lg, N - 1);  // this lane's channel (clamped: results past N unused)
  unsigned char* xw = lds + (size_t)kw * R * a.slice;                             // [R][slice]
  float* part = reinterpret_cast<float*>(lds + (size_t)kWaves * R * a.slice);     // [4][R][8]
  float* scl = part + (size_t)kWaves * R * 8;                                     // [R][8]
  int32_t* c_row = reinterpret_cast<int32_t*>(scl + (I8 ? (size_t)R * 8 : 0));   // [T * k]
  float* c_w = reinterpret_cast<float*>(c_row + Tk);                             // [T * k]

  // (0) the combine's inputs, loaded now and used at the end: one routed slot per thread,
  //     and the residual of thread (token tid / 8, channel tid % 8)
  int my_row = -1;
  float my_w = 0.f;
  if (tid < Tk) {
    my_row = a.inv_perm[tid];
    my_w = a.topk_w[tid];
  }
  const int ct = tid / 8, cn = n0 + tid % 8;
  // raw and unconditional (a thread past the tokens, or no residual, reads an in-bounds
  // element it ignores), so the load is only waited for where the value is used, at the end
  const AT* rsrc = a.residual ? reinterpret_cast<const AT*>(a.residual) + (size_t)min(ct, T - 1) * N + min(cn, N - 1)
                              : reinterpret_cast<const AT*>(a.h);
  const AT resid = *rsrc;

  // (1) K-slice kw of every row into its LDS region, shared by the NG wavefronts of that
  //     slice (64 pieces each in turn): piece c of the region is row c / cpr, 16 bytes at
  //     column kw0 + (c % cpr) * 16 / sizeof(AT)
  const int steps = (K + STEP - 1) / STEP;
  const int spw = a.slice / (STEP * (int)sizeof(AT));
  const int s_lo = kw * spw, s_hi = min(steps, s_lo + spw);
  const int kw0 = s_lo * STEP;
  const AT* h = reinterpret_cast<const AT*>(a.h);
  if (s_lo < steps) {
    const int cpr = a.slice / 16;
    const int dr = NG * kWave / cpr, dp = NG * kWave % cpr;  // (row, piece) advance per turn
    int r = (grp * kWave + lane) / cpr, p = (grp * kWave + lane) % cpr;
    for (int c0 = grp * kWave; c0 < R * cpr; c0 += NG * kWave) {
      int col = kw0 + p * (16 / (int)sizeof(AT));
      if (col >= K) col = kw0;  // the last wavefront's slice past K: an in-bounds piece, never read
      if (r < R)
        __builtin_amdgcn_global_load_lds((gmem_void*)(h + (size_t)r * K + col), (lds_void*)(xw + c0 * 16),
                                         16, 0, 0);
      r += dr;
      p += dp;
      if (p >= cpr) {
        p -= cpr;
        ++r;
      }
    }
  }

  // (2) the weight ring over the touched groups: slot stream grp takes groups grp, grp + NG, ...
  const cint32* plan = (const cint32*)a.plan;
  const cint32* offs = (const cint32*)a.offsets;
  const WT* wbase = reinterpret_cast<const WT*>(a.w);
  const int nslots = plan[0], cap = plan[3];
  const int mine = nslots > grp ? (nslots - grp + NG - 1) / NG : 0;  // this stream's groups
  uint4 wb[D][MAXIT];
  float sc[D];
  auto issue = [&](int i, int j) {
    const int g = plan[kPlanHeader + grp + i * NG];
    const WT* wp = wbase + ((size_t)g * N + n) * K;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
      const int col = kw0 + it * STEP + q * V;
      const int colc = (s_lo + it < s_hi && col < K) ? col : (q * V < K ? q * V : 0);
      wb[j][it] = *reinterpret_cast<const uint4*>(wp + colc);
    }
    if (I8) sc[j] = a.s[(size_t)g * N + n];
  };
  auto process = [&](int i, int j) {
    const int g = plan[kPlanHeader + grp + i * NG];
    const int r0 = offs[g];
    const int Mg = offs[g + 1] - r0;
    const int M = (g < a.E && cap > 0) ? min(Mg, cap) : Mg;  // capacity: the rest is dropped
    for (int m0 = 0; m0 < M; m0 += MB) {
      float acc[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[m] = 0.f;
#pragma unroll
      for (int it = 0; it < MAXIT; ++it) {
        const int xcol = it * STEP + q * V;  // column within the slice
        if (s_lo + it < s_hi && kw0 + xcol < K) {
          const typename Dt::W wv = Dt::prep(wb[j][it]);
          const unsigned char* xp = xw + (size_t)(r0 + m0) * a.slice + xcol * (int)sizeof(AT);
#pragma unroll
          for (int m = 0; m < MB; ++m)
            if (m0 + m < M) acc[m] = Dt::run(wv, xp + m * a.slice, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float v = sum8(settle_dot(acc[m]));
        if (m0 + m < M && q == (m & 7)) {
          const int r = r0 + m0 + m;
          part[((size_t)kw * R + r) * 8 + lg] = v;
          if (I8 && kw == 0) scl[(size_t)r * 8 + lg] = sc[j];
        }
      }
    }
  };
  if (mine > 0) {
#pragma unroll
    for (int j = 0; j < D; ++j) issue(min(j, mine - 1), j);
  }
  // the staged rows are in and visible to every wavefront (this also waits for the first
  // groups' weights, which their sums needed anyway; direct-to-LDS loads are not ordered with
  // the register loads behind them, so no partial wait would do)
  __syncthreads();
  if (mine > 0) {
    for (int i0 = 0; i0 < mine; i0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (i0 + j < mine) process(i0 + j, j);
        issue(min(i0 + j + D, mine - 1), j);
      }
    }
  }

  // (3) every wavefront's partial sums are in: each thread (token, channel) sums the token's
  //     rows in the combine's order
  if (tid < Tk) {
    c_row[tid] = my_row;
    c_w[tid] = my_w;
  }
  __syncthreads();
  if (ct < T && cn < N) {
    const int c = tid % 8;
    auto row = [&](int r) {
      float v = (part[(size_t)r * 8 + c] + part[((size_t)R + r) * 8 + c]) +
                (part[((size_t)2 * R + r) * 8 + c] + part[((size_t)3 * R + r) * 8 + c]);
      if (I8) v *= scl[(size_t)r * 8 + c];
      return Act<AT>::round(v);
    };
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = c_row[ct * k + j];
      if (r >= 0) acc = fmaf(c_w[ct * k + j], row(r), acc);
    }
    for (int sx = 0; sx < a.S; ++sx) acc = acc + row(Tk + sx * T + ct);
    if (a.residual) acc = acc + Act<AT>::load(&resid, 0);
    Act<AT>::store(reinterpret_cast<AT*>(a.y), (size_t)ct * N + cn, acc);
  }
}

template <typename AT, typename WT, int MB>
hipError_t run_down_combine(const DownCombineArgs& a, int spw, size_t lds, hipStream_t s) {
  constexpr int NG = dc_streams<WT>();
  switch (spw) {
#define DC_CASE(MAXIT)                                                                             \
  case MAXIT: {                                                                                     \
    static LdsFlags done;                                                                           \
    hipError_t e = set_lds(&k_down_combine<AT, WT, MAXIT, MB, NG>, kDcMaxLds, done);               \
    if (e != hipSuccess) return e;                                                                  \
    /* the combine's hook brackets the launch it shares with the down projection */                \
    LaunchTimer combine_timer(MOE_KERNEL_COMBINE, s);                                              \
    return launch(MOE_KERNEL_DOWN, k_down_combine<AT, WT, MAXIT, MB, NG>, dim3((a.N + 7) / 8), 256 * NG, \
                  lds, s, a);                                                                       \
  }
    DC_CASE(1)
    DC_CASE(2)
    DC_CASE(3)
    DC_CASE(4)
    DC_CASE(5)
    DC_CASE(6)
    DC_CASE(7)
    DC_CASE(8)
#undef DC_CASE
    default: return hipErrorInvalidValue;
  }
}

template <typename AT, typename WT>
hipError_t dispatch_down_combine(const DownCombineArgs& a, int spw, size_t lds, hipStream_t s) {
  return a.T == 1 ? run_down_combine<AT, WT, 1>(a, spw, lds, s) : run_down_combine<AT, WT, 4>(a, spw, lds, s);
}
}  // namespace

namespace {
GemvArgs gemv_args(const LayerDims& L, const FfnArgs& f) {
  GemvArgs a{};
  a.offsets = f.offsets;
  a.perm = f.perm;
  a.plan = f.plan;
  a.k = L.k;
  a.E = L.E;
  return a;
}

// gate/up + SwiGLU on the VALU GEMV
hipError_t gemv_gate_up(const LayerDims& L, int T, const FfnArgs& f, hipStream_t s) {
  const int slots = (T * L.k < L.E ? T * L.k : L.E) + L.S;
  GemvArgs a = gemv_args(L, f);
  a.in = f.x;
  a.w0 = f.w_gate;
  a.w1 = f.w_up;
  a.s0 = f.s_gate;
  a.s1 = f.s_up;
  a.out = f.h;
  a.K = L.d;
  a.N = L.I;
  if (L.act == MOE_F32) return dispatch_gemv<0, float, float>(a, T, slots, s);
  if (L.wdt == MOE_I8) return dispatch_gemv<0, uint16_t, int8_t>(a, T, slots, s);
  return dispatch_gemv<0, uint16_t, uint16_t>(a, T, slots, s);
}

// The fused launch's geometry: K steps per wavefront, a row's wavefront slice in LDS, the
// rows, and the LDS it takes (staged rows, partial sums, int8 scales, the combine's slots).
struct DownCombineGeom {
  int spw, slice, R;
  size_t lds;
};
DownCombineGeom down_combine_geom(const LayerDims& L, int T) {
  const bool f32 = L.act == MOE_F32, i8 = L.wdt == MOE_I8;
  const int V = f32 ? 4 : (i8 ? 16 : 8), esz = f32 ? 4 : 2;
  const int steps = (L.I + 8 * V - 1) / (8 * V);
  DownCombineGeom g;
  g.spw = (steps + kWaves - 1) / kWaves;
  g.slice = g.spw * 8 * V * esz;
  g.R = T * L.k + L.S * T;
  g.lds = (size_t)kWaves * g.R * g.slice + (size_t)kWaves * g.R * 8 * 4 + (i8 ? (size_t)g.R * 8 * 4 : 0) +
          (size_t)T * L.k * 8;
  return g;
}
}  // namespace

bool gemv_down_combine_fits(const LayerDims& L, int T) {
  const DownCombineGeom g = down_combine_geom(L, T);
  // (int8 past 6 steps per wavefront would spill registers at four slot streams)
  const int max_spw = L.wdt == MOE_I8 ? 6 : 8;
  return T >= 1 && T * 8 <= 256 && T * L.k <= 256 && g.spw <= max_spw && g.lds <= kDcMaxLds;
}

hipError_t launch_gemv_ffn(const LayerDims& L, int T, const FfnArgs& f, hipStream_t s) {
  hipError_t err = gemv_gate_up(L, T, f, s);
  if (err != hipSuccess) return err;
  const int slots = (T * L.k < L.E ? T * L.k : L.E) + L.S;
  GemvArgs a = gemv_args(L, f);
  a.in = f.h;
  a.w0 = f.w_down;
  a.w1 = nullptr;
  a.s0 = f.s_down;
  a.s1 = nullptr;
  a.out = f.rows;
  a.K = L.I;
  a.N = L.d;
  if (L.act == MOE_F32) return dispatch_gemv<1, float, float>(a, T, slots, s);
  if (L.wdt == MOE_I8) return dispatch_gemv<1, uint16_t, int8_t>(a, T, slots, s);
  return dispatch_gemv<1, uint16_t, uint16_t>(a, T, slots, s);
}

hipError_t launch_gemv_ffn_combine(const LayerDims& L, int T, const FfnArgs& f, const int32_t* inv_perm,
                                   const float* topk_w, const void* residual, void* y, hipStream_t s) {
  if (!gemv_down_combine_fits(L, T)) return hipErrorInvalidValue;
  hipError_t err = gemv_gate_up(L, T, f, s);
  if (err != hipSuccess) return err;
  const DownCombineGeom g = down_combine_geom(L, T);
  DownCombineArgs a{f.h, f.w_down, f.s_down, f.offsets, f.plan, inv_perm, topk_w, residual, y,
                    T, L.k, L.S, L.E, L.I, L.d, g.R, g.slice};
  if (L.act == MOE_F32) return dispatch_down_combine<float, float>(a, g.spw, g.lds, s);
  if (L.wdt == MOE_I8) return dispatch_down_combine<uint16_t, int8_t>(a, g.spw, g.lds, s);
  return dispatch_down_combine<uint16_t, uint16_t>(a, g.spw, g.lds, s);
}

hipError_t launch_gemv_mfma_ffn(const LayerDims& L, int T, const FfnArgs& f, hipStream_t s) {
  if (L.act != MOE_BF16 || L.d % 64 != 0 || L.I % 64 != 0) return hipErrorInvalidValue;
  const int slots = (T * L.k < L.E ? T * L.k : L.E) + L.S;
  const bool i8 = L.wdt == MOE_I8;
  GemvArgs a{};
  a.offsets = f.offsets;
  a.perm = f.perm;
  a.plan = f.plan;
  a.k = L.k;
  a.E = L.E;

  // gate/up + SwiGLU
  a.in = f.x;
  a.w0 = f.w_gate;
  a.w1 = f.w_up;
  a.s0 = f.s_gate;
  a.s1 = f.s_up;
  a.out = f.h;
  a.K = L.d;
  a.N = L.I;
  hipError_t err = i8 ? dispatch_gemv_mfma<0, true>(a, slots, s) : dispatch_gemv_mfma<0, false>(a, slots, s);
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
  return i8 ? dispatch_gemv_mfma<1, true>(a, slots, s) : dispatch_gemv_mfma<1, false>(a, slots, s);
}

}  // namespace moe
