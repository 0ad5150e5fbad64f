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
          const float v = sum8(acc[c][t][m]);
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

  // gate/up + SwiGLU
  a.in = f.x;
  a.w0 = f.w_gate;
  a.w1 = f.w_up;
  a.s0 = f.s_gate;
  a.s1 = f.s_up;
  a.out = f.h;
  a.K = L.d;
  a.N = L.I;
  if (L.act == MOE_F32)
    err = dispatch_gemv<0, float, float>(a, T, slots, s);
  else if (L.wdt == MOE_I8)
    err = dispatch_gemv<0, uint16_t, int8_t>(a, T, slots, s);
  else
    err = dispatch_gemv<0, uint16_t, uint16_t>(a, T, slots, s);
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
  if (L.act == MOE_F32)
    err = dispatch_gemv<1, float, float>(a, T, slots, s);
  else if (L.wdt == MOE_I8)
    err = dispatch_gemv<1, uint16_t, int8_t>(a, T, slots, s);
  else
    err = dispatch_gemv<1, uint16_t, uint16_t>(a, T, slots, s);
  return err;
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
