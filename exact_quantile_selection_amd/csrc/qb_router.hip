// qb_router.hip -- router GEMM on MFMA for the fused-router workload:
// logits[N][E] = hidden[N][H] . w[E][H]^T (bf16 inputs, fp32 accumulation),
// s = sigmoid(logits) written as the fp32 score matrix the balancing passes
// read.  The router's forward ("[Dev] Add global-batch quantile balancing",
// Megatron-LM PR #6637, Validation: real router forward/backward) produces
// the sigmoid scores of section "Quantile estimator".
//
// The op streams `hidden` (2H bytes per token) and writes s (4E bytes per
// token); at E = 256, H = 2048 that is 1.34 GB against 2.75e11 flop, below
// MI355X's ridge, so HBM bounds it once the matrix cores keep up:
//
//  * one workgroup of 8 waves (2 per SIMD) owns 256 token rows and all E
//    expert columns, so each token row is read from HBM once and the weight
//    (2EH bytes, L2-resident) is re-read once per 256 rows;
//  * waves tile the 256 x E block as WAVES_M x WAVES_N, each holding a
//    (32 TM) x (32 TN) sub-block in TM * TN accumulators of
//    v_mfma_f32_32x32x16_bf16 (64 x 128 per wave at E = 256, so each LDS
//    operand fragment feeds 4 or 2 MFMAs);
//  * K advances in tiles of BK through an S-deep ring of LDS stages filled
//    by global_load_lds_dwordx4 (memory -> LDS without registers), S - 1
//    tiles ahead of the multiply; one barrier per tile;
//  * each LDS tile is a sequence of 256-byte lines of sixteen 16-byte slots
//    (gfx950's LDS serves a 16-byte read for 16 lanes per cycle across 64
//    banks); a tile row holds BK/8 chunks, and the chunk bits of the slot
//    index are XORed with (line mod BK/8), so the 16 lanes of a phase --
//    16 consecutive rows at one chunk -- land on 16 distinct slots.  The
//    loads place lane l's 16 bytes at the l-th slot of the instruction's
//    1 KiB, so the swizzle is applied by choosing which global chunk each
//    lane fetches.
//
// MFMA 32x32x16 bf16 operand layout (checked on the GPU): lane l supplies
// A[row = l % 32][k = 8 * (l / 32) + j] and B[k = 8 * (l / 32) + j][col = l % 32],
// j = 0..7; result element i of lane l is C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32].
#include <algorithm>

#include "qb_device.hpp"
#include "qb_internal.hpp"

#ifndef QB_RG_BK
#define QB_RG_BK 64
#endif
#ifndef QB_RG_STAGES
#define QB_RG_STAGES 2
#endif

namespace qbk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(1))) void* glb_vptr;

#ifndef QB_RG_WAVES
#define QB_RG_WAVES 8
#endif
constexpr int kRgWaves = QB_RG_WAVES;
constexpr int kRgThreads = kRgWaves * kWave;
constexpr int kRgBM = 32 * kRgWaves;  // token rows per workgroup

template <int E>
struct RgShape {
  static constexpr int WAVES_N = E >= 64 ? 2 : 1;
  static constexpr int WAVES_M = kRgWaves / WAVES_N;
  static constexpr int TM = kRgBM / 32 / WAVES_M;  // 32-row tiles per wave
  static constexpr int TN = E / 32 / WAVES_N;      // 32-column tiles per wave
  static_assert(WAVES_M * TM * 32 == kRgBM && WAVES_N * TN * 32 == E, "tiling");
};

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int rg_vmcnt(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

// Physical 16-byte slot of logical chunk q (= row * CPR + chunk) inside a
// tile: lines of 16 slots, chunk bits XOR (line mod CPR).  An involution.
template <int CPR>
__device__ __forceinline__ int rg_phys(int q) { return q ^ ((q >> 4) & (CPR - 1)); }

// sigmoid(x) = 1 / (1 + 2^(-x log2 e)).  The exponent is reduced in the
// manner of Cody and Waite: t = -x log2 e is carried as hi + lo (log2 e
// split into a float and its remainder, the product's rounding error
// recovered exactly with an FMA), n = rint(hi), f = (hi - n) + lo with
// |f| <= 1/2, and 2^t = ldexp(2^f, n) with 2^f from v_exp_f32.  The
// reciprocal is v_rcp_f32.  x is clamped to [-128, 128], where fp32
// sigmoid is already 0 (below about -87.3 the result is flushed to 0) or 1,
// so infinities behave; NaN logits give an unspecified score.
__device__ __forceinline__ float rg_sigmoid(float x) {
  constexpr float kLog2eHi = 1.44269502162933349609375f;   // fl32(log2 e)
  constexpr float kLog2eLo = 1.925963033500011079e-8f;     // fl32(log2 e - kLog2eHi)
  x = __builtin_amdgcn_fmed3f(x, -128.0f, 128.0f);
  const float hi = -x * kLog2eHi;
  const float lo = fmaf(-x, kLog2eLo, fmaf(-x, kLog2eHi, -hi));
  const float n = rintf(hi);
  const float f = (hi - n) + lo;
  const float e = __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(f), int(n));
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Pass 1 in the GEMM epilogue ("[Dev] Add global-batch quantile balancing",
// section "Implementation": the fused routing path adds bin classification
// and histogram atomics in shared memory to the router kernel; section
// "Quantile estimator": alpha, the margins; "Exact Quantile Balancing and
// Load-Error Injection for Mixture-of-Experts", EQB paragraph: the
// high-byte histogram of the bf16 margins).
//
// After the K loop a token's E scores sit in four places (two lanes of each
// of two waves).  The workgroup has just stored its 256 rows of scores, so
// once its waves meet at a barrier it reads them back, still in L2, row by
// row: each row by LPR = E/32 lanes holding 32 scores each, in the layout of
// the standalone pass 1 -- top-(K+1) of s + b by v_med3 insertion and DPP
// merges (quad xor 1, quad xor 2, half-row mirror), alpha, the top-K loads
// and the high-byte key histogram.  (Passing the scores through LDS instead
// keeps the 128 accumulators live beside the row state and spills.)
//
// The high-byte histogram is counted in LDS with the standalone pass's packed
// 16-bit counters (E x 512 bytes: 128 KiB at E = 256, in the LDS the operand
// ring used) and flushed once per workgroup, one 64-bit device atomic per two
// adjacent bins.  Each lane keeps the rows of two steps in flight.
template <int E>
struct RfShape {
  static constexpr int LPR = E / 32;                       // lanes per row
  static constexpr int F4 = 8;                             // float4 per lane (32 scores)
  static constexpr int RPW = kWave / LPR;                  // rows per wave and step
  static constexpr int R = kRgWaves * RPW < kRgBM ? kRgWaves * RPW : kRgBM;  // rows per step
  static constexpr int WAVES_USED = R / RPW;
  static constexpr int NP = kRgBM / R;                     // steps per workgroup
  static constexpr int HIST_BYTES = E * 512;
  static constexpr int BIAS_OFF = HIST_BYTES;
  static constexpr int LOAD_OFF = BIAS_OFF + E * 4;
  static constexpr int BYTES = LOAD_OFF + E * 4;
  static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8, "lanes per row");
  static_assert(kRgBM % R == 0, "steps");
};


template <int P, int LPR>
__device__ __forceinline__ void rf_merge_rows(float (&t)[P]) {
  if constexpr (LPR >= 2) top_merge<P, kQuadXor1>(t);
  if constexpr (LPR >= 4) top_merge<P, kQuadXor2>(t);
  if constexpr (LPR >= 8) top_merge<P, kHalfMirror>(t);
}

template <int LPR>
__device__ __forceinline__ int rf_row_sum(int x) {
  if constexpr (LPR >= 2) x += quad_mov_i<kQuadXor1>(x);
  if constexpr (LPR >= 4) x += quad_mov_i<kQuadXor2>(x);
  if constexpr (LPR >= 8) x += quad_mov_i<kHalfMirror>(x);
  return x;
}

template <int E, int P>
__device__ __forceinline__ void rf_epilogue(uint8_t* lds, int lane, int wave, int tid, int64_t m0, int64_t N,
                                            const float* s_rows, const float* bias, int K, float* alpha,
                                            int32_t* load, int32_t* hist_hi) {
  using F = RfShape<E>;
  constexpr int LPR = F::LPR;
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds);
  float* lds_b = reinterpret_cast<float*>(lds + F::BIAS_OFF);
  int32_t* lds_load = reinterpret_cast<int32_t*>(lds + F::LOAD_OFF);
  const bool want_hist = hist_hi != nullptr, want_load = load != nullptr;

  if (want_hist) hist16_zero<E>(hist, tid, kRgThreads);
  for (int j = tid; j < E; j += kRgThreads) {
    lds_b[j] = bias[j];
    lds_load[j] = 0;
  }
  // the barrier publishes the LDS set-up and this workgroup's score stores
  __syncthreads();
  const int rho = lane / LPR, ql = lane % LPR;
  if (wave < F::WAVES_USED) {
    // rows of up to two steps in flight: step p + 2 is loaded once step p
    // has been ranked
    constexpr int NB = F::NP < 2 ? F::NP : 2;
    float4 xb[NB][F::F4];
    auto fetch = [&](int p, float4(&x)[F::F4]) {
      const int64_t row = m0 + int64_t(p) * F::R + wave * F::RPW + rho;
      const float* src = s_rows + (row < N ? row : N - 1) * E;
#pragma unroll
      for (int t = 0; t < F::F4; ++t) x[t] = ld4(src + 4 * (LPR * ((t + rho) & (F::F4 - 1)) + ql));
    };
#pragma unroll
    for (int p = 0; p < NB; ++p) fetch(p, xb[p]);
#pragma unroll
    for (int p = 0; p < F::NP; ++p) {
      float4(&xp)[F::F4] = xb[p % NB];
      const int64_t row = m0 + int64_t(p) * F::R + wave * F::RPW + rho;
      const bool valid = row < N;
      float top[P];
#pragma unroll
      for (int k = 0; k < P; ++k) top[k] = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < F::F4; ++t) {
        const int Q = LPR * ((t + rho) & (F::F4 - 1)) + ql;
        const float4 bb = *reinterpret_cast<const float4*>(lds_b + 4 * Q);
        top_insert<P>(top, xp[t].x + bb.x);
        top_insert<P>(top, xp[t].y + bb.y);
        top_insert<P>(top, xp[t].z + bb.z);
        top_insert<P>(top, xp[t].w + bb.w);
      }
      rf_merge_rows<P, LPR>(top);
      float a = top[0];
#pragma unroll
      for (int k = 1; k < P; ++k) a = k == K ? top[k] : a;
      if (valid && ql == 0) __builtin_nontemporal_store(a, alpha + row);
      if (want_load) {
        // members: v > alpha, plus the lowest-index elements equal to alpha
        // up to K in all.  Bit 4u + c of a lane's masks is its element of
        // expert 4 (LPR u + ql) + c, so bit order is expert order.
        uint32_t gt = 0;
#pragma unroll
        for (int t = 0; t < F::F4; ++t) {
          const int u = (t + rho) & (F::F4 - 1);
          const float4 bb = *reinterpret_cast<const float4*>(lds_b + 4 * (LPR * u + ql));
          gt |= (xp[t].x + bb.x > a ? 1u : 0u) << (4 * u);
          gt |= (xp[t].y + bb.y > a ? 1u : 0u) << (4 * u + 1);
          gt |= (xp[t].z + bb.z > a ? 1u : 0u) << (4 * u + 2);
          gt |= (xp[t].w + bb.w > a ? 1u : 0u) << (4 * u + 3);
        }
        uint32_t mem = gt;
        const int need = K - rf_row_sum<LPR>(__popc(gt));
        if (__ballot(valid && need > 0) != 0) {  // a tie at alpha somewhere in the wave
          uint32_t eq = 0;
#pragma unroll
          for (int t = 0; t < F::F4; ++t) {
            const int u = (t + rho) & (F::F4 - 1);
            const float4 bb = *reinterpret_cast<const float4*>(lds_b + 4 * (LPR * u + ql));
            eq |= (xp[t].x + bb.x == a ? 1u : 0u) << (4 * u);
            eq |= (xp[t].y + bb.y == a ? 1u : 0u) << (4 * u + 1);
            eq |= (xp[t].z + bb.z == a ? 1u : 0u) << (4 * u + 2);
            eq |= (xp[t].w + bb.w == a ? 1u : 0u) << (4 * u + 3);
          }
          uint32_t M[LPR];
#pragma unroll
          for (int q2 = 0; q2 < LPR; ++q2) M[q2] = __shfl(eq, rho * LPR + q2);
          if (valid && need > 0) {
            uint32_t e = eq;
            while (e) {
              const int bit = __builtin_ctz(e);
              e &= e - 1;
              const int u = bit >> 2, c = bit & 3;
              int rank = 0;
#pragma unroll
              for (int q2 = 0; q2 < LPR; ++q2) {
                const int nb = q2 < ql ? 4 * (u + 1) : (q2 > ql ? 4 * u : 4 * u + c);
                rank += __popc(M[q2] & (nb >= 32 ? 0xFFFFFFFFu : ((1u << nb) - 1u)));
              }
              if (rank < need) mem |= 1u << bit;
            }
          }
        }
        if (valid) {
          while (mem) {
            const int bit = __builtin_ctz(mem);
            mem &= mem - 1;
            atomicAdd(&lds_load[4 * (LPR * (bit >> 2) + ql) + (bit & 3)], 1);
          }
        }
      }
      if (want_hist && valid) {
#pragma unroll
        for (int t = 0; t < F::F4; ++t) {
          const int Q = LPR * ((t + rho) & (F::F4 - 1)) + ql;
          const uint32_t swz = hist16_swizzle2(Q);
          hist16_add_hi(hist, Q, 0, key2(bf16x2_rne(a - xp[t].x, a - xp[t].y)) ^ swz);
          hist16_add_hi(hist, Q, 2, key2(bf16x2_rne(a - xp[t].z, a - xp[t].w)) ^ swz);
        }
      }
      if (p + NB < F::NP) fetch(p + NB, xp);
    }
  }
  __syncthreads();
  if (want_hist) hist16_flush_pairs<E>(hist, hist_hi, tid, kRgThreads, int(blockIdx.x));
  if (want_load)
    for (int j = tid; j < E; j += kRgThreads)
      if (lds_load[j]) atomicAdd(load + j, lds_load[j]);
}

template <int E, int BK, int S, int P>
__global__ __launch_bounds__(kRgThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_router_gemm(const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w, int64_t N, int H,
                   float* __restrict__ s_out, float* __restrict__ logits_out, const float* __restrict__ bias,
                   int K, float* __restrict__ alpha, int32_t* __restrict__ load, int32_t* __restrict__ hist_hi) {
  using Sh = RgShape<E>;
  constexpr int TM = Sh::TM, TN = Sh::TN;
  constexpr int CPR = BK / 8;                        // 16-byte chunks per tile row
  constexpr int A_BYTES = kRgBM * BK * 2;
  constexpr int B_BYTES = E * BK * 2;
  constexpr int A_INSTR = kRgBM * CPR / kWave;      // 1 KiB load instructions per A tile
  constexpr int B_INSTR = E * CPR / kWave;
  constexpr int A_PER_WAVE = A_INSTR / kRgWaves;
  constexpr int B_PER_WAVE = (B_INSTR + kRgWaves - 1) / kRgWaves;
  constexpr int PER_STAGE = A_PER_WAVE + B_PER_WAVE;  // loads per wave per stage
  static_assert(A_INSTR % kRgWaves == 0, "A tile split");
  static_assert(BK % 16 == 0 && CPR <= 16 && 16 % CPR == 0, "BK");
  constexpr int RING_BYTES = S * (A_BYTES + B_BYTES);
  constexpr int LDS_BYTES = P == 0 ? RING_BYTES
                                   : (RING_BYTES > RfShape<E>::BYTES ? RING_BYTES : RfShape<E>::BYTES);
  __shared__ __align__(1024) uint8_t lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / Sh::WAVES_N, wn = wave % Sh::WAVES_N;
  const int64_t m0 = int64_t(blockIdx.x) * kRgBM;
  const int KT = H / BK;

  // Per-lane global sources of this wave's load instructions (tile 0); the
  // k offset advances by BK per tile.  Rows past N re-read row N - 1.
  const uint16_t* a_src[A_PER_WAVE];
#pragma unroll
  for (int j = 0; j < A_PER_WAVE; ++j) {
    const int p = (wave * A_PER_WAVE + j) * kWave + lane;  // physical slot
    const int q = rg_phys<CPR>(p);                               // logical chunk (involution)
    int64_t row = m0 + q / CPR;
    row = row < N ? row : N - 1;
    a_src[j] = hidden + row * H + (q % CPR) * 8;
  }
  const uint16_t* b_src[B_PER_WAVE];
  int b_slot[B_PER_WAVE];
#pragma unroll
  for (int j = 0; j < B_PER_WAVE; ++j) {
    const int g = (wave * B_PER_WAVE + j) % B_INSTR;  // extra waves repeat a load
    const int q = rg_phys<CPR>(g * kWave + lane);
    b_src[j] = w + int64_t(q / CPR) * H + (q % CPR) * 8;
    b_slot[j] = g;
  }

  // Workgroup b walks the K tiles starting at tile b mod KT: the workgroups
  // in flight then read different column offsets of their rows, which
  // spreads their requests over the HBM channels (streaming `hidden` alone,
  // without the matrix work, took 255 us in K order and 186 us rotated; the
  // whole kernel 413-421 against 410-412 us).  The fp32 sums run in a
  // rotated order; the scores stay within the same tolerance.
  const int krot = int(blockIdx.x % unsigned(KT));
  auto issue = [&](int kt) {
    uint8_t* sa = lds + (kt % S) * A_BYTES;
    uint8_t* sb = lds + S * A_BYTES + (kt % S) * B_BYTES;
    const int kr = kt + krot;
    const int koff = (kr < KT ? kr : kr - KT) * BK;
#pragma unroll
    for (int j = 0; j < A_PER_WAVE; ++j)
      __builtin_amdgcn_global_load_lds((glb_vptr)(a_src[j] + koff),
                                       (lds_vptr)(sa + (wave * A_PER_WAVE + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < B_PER_WAVE; ++j)
      __builtin_amdgcn_global_load_lds((glb_vptr)(b_src[j] + koff), (lds_vptr)(sb + b_slot[j] * 1024),
                                       16, 0, 0);
  };

  // LDS byte offsets of this lane's operand fragments inside a stage.
  int a_off[TM][BK / 16], b_off[TN][BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = ks * 2 + lane / 32;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      a_off[tm][ks] = rg_phys<CPR>(((wm * TM + tm) * 32 + lane % 32) * CPR + c) * 16;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      b_off[tn][ks] = rg_phys<CPR>(((wn * TN + tn) * 32 + lane % 32) * CPR + c) * 16;
  }

  floatx16 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tm][tn][i] = 0.0f;

#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < KT) issue(t);

  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of tile kt are done once at most the later tiles'
    // loads are outstanding; the barrier then publishes every wave's tile
    // and retires all reads of the stage the next issue overwrites
    if (kt + S - 2 < KT)
      __builtin_amdgcn_s_waitcnt(rg_vmcnt((S - 2) * PER_STAGE));
    else
      __builtin_amdgcn_s_waitcnt(rg_vmcnt(0));
    // bare barrier: the wait above already covers this wave's tile, and every
    // LDS read of the previous tile has been consumed by its MFMAs.  A
    // __syncthreads() (or any LDS release fence) would wait for all pending
    // memory->LDS loads and drain the ring.  The empty asm statements keep
    // the compiler from moving LDS accesses across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + S - 1 < KT) issue(kt + S - 1);
    const uint8_t* sa = lds + (kt % S) * A_BYTES;
    const uint8_t* sb = lds + S * A_BYTES + (kt % S) * B_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) a[tm] = *reinterpret_cast<const bf16x8*>(sa + a_off[tm][ks]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) b[tn] = *reinterpret_cast<const bf16x8*>(sb + b_off[tn][ks]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[tn], a[tm], acc[tm][tn], 0, 0, 0);
    }
  }

  // epilogue: sigmoid, store scores (and logits on request).  The weight
  // fragment is the MFMA's first operand, so acc[tm][tn] holds the
  // transposed tile, experts x tokens: element 4 q + c of lane l is expert
  // 8 q + 4 (l / 32) + c of token l % 32, and each lane stores four
  // consecutive scores of one token with one 16-byte store (a quarter of
  // the store instructions of the token-major layout; 410-412 against
  // 417-422 us at 262,144 x 2048 x 256, the same scores bit for bit).
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t row = m0 + (wm * TM + tm) * 32 + (lane % 32);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = (wn * TN + tn) * 32 + 8 * q + 4 * (lane / 32);
        if (logits_out && row < N) {  // 4-byte aligned only
          float* lo = logits_out + row * E + col;
          lo[0] = acc[tm][tn][4 * q];
          lo[1] = acc[tm][tn][4 * q + 1];
          lo[2] = acc[tm][tn][4 * q + 2];
          lo[3] = acc[tm][tn][4 * q + 3];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[tm][tn][4 * q + c] = rg_sigmoid(acc[tm][tn][4 * q + c]);
        if (row < N)
          *reinterpret_cast<float4*>(s_out + row * E + col) =
              make_float4(acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2],
                          acc[tm][tn][4 * q + 3]);
      }
  }
  if constexpr (P > 0) {
    // every wave is past its last LDS read of the ring
    __syncthreads();
    rf_epilogue<E, P>(lds, lane, wave, tid, m0, N, s_out, bias, K, alpha, load, hist_hi);
  }
}

template <int E, int P>
static int launch_rg(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, float* s_out,
                     float* logits_out, const float* b, int K, float* alpha, int32_t* load, int32_t* hist_hi,
                     hipStream_t st) {
  const dim3 grid{unsigned((N + kRgBM - 1) / kRgBM), 1u, 1u};
  const dim3 block{unsigned(kRgThreads), 1u, 1u};
  hipLaunchKernelGGL((k_router_gemm<E, QB_RG_BK, QB_RG_STAGES, P>), grid, block, 0, st, hidden, w, N, H, s_out,
                     logits_out, b, K, alpha, load, hist_hi);
  return int(hipGetLastError());
}

int launch_router_gemm(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                       float* s_out, float* logits_out, hipStream_t st) {
  switch (E) {
    case 32: return launch_rg<32, 0>(hidden, w, N, H, s_out, logits_out, nullptr, 0, nullptr, nullptr, nullptr, st);
    case 64: return launch_rg<64, 0>(hidden, w, N, H, s_out, logits_out, nullptr, 0, nullptr, nullptr, nullptr, st);
    case 128:
      return launch_rg<128, 0>(hidden, w, N, H, s_out, logits_out, nullptr, 0, nullptr, nullptr, nullptr, st);
    case 256:
      return launch_rg<256, 0>(hidden, w, N, H, s_out, logits_out, nullptr, 0, nullptr, nullptr, nullptr, st);
    default: return int(hipErrorInvalidValue);
  }
}

template <int P>
static int launch_rf_p(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E, float* s_out,
                       float* logits_out, const float* b, int K, float* alpha, int32_t* load, int32_t* hist_hi,
                       hipStream_t st) {
  switch (E) {
    case 32: return launch_rg<32, P>(hidden, w, N, H, s_out, logits_out, b, K, alpha, load, hist_hi, st);
    case 64: return launch_rg<64, P>(hidden, w, N, H, s_out, logits_out, b, K, alpha, load, hist_hi, st);
    case 128: return launch_rg<128, P>(hidden, w, N, H, s_out, logits_out, b, K, alpha, load, hist_hi, st);
    case 256: return launch_rg<256, P>(hidden, w, N, H, s_out, logits_out, b, K, alpha, load, hist_hi, st);
    default: return int(hipErrorInvalidValue);
  }
}

// Router GEMM with pass 1 in its epilogue: lists of 8 for K <= 7, of 16 up
// to K = 15.
int launch_router_fused(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E, float* s_out,
                        float* logits_out, const float* b, int K, float* alpha, int32_t* load, int32_t* hist_hi,
                        hipStream_t st) {
  if (K + 1 <= 8) return launch_rf_p<8>(hidden, w, N, H, E, s_out, logits_out, b, K, alpha, load, hist_hi, st);
  return launch_rf_p<16>(hidden, w, N, H, E, s_out, logits_out, b, K, alpha, load, hist_hi, st);
}

}  // namespace qbk
