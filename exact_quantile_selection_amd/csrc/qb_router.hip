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

template <int E, int BK, int S>
__global__ __launch_bounds__(kRgThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_router_gemm(const uint16_t* __restrict__ hidden,
                                                            const uint16_t* __restrict__ w,
                                                            int64_t N, int H,
                                                            float* __restrict__ s_out,
                                                            float* __restrict__ logits_out) {
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
  __shared__ __align__(1024) uint8_t lds[S * (A_BYTES + B_BYTES)];

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
    if (row >= N) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = (wn * TN + tn) * 32 + 8 * q + 4 * (lane / 32);
        const float x0 = acc[tm][tn][4 * q], x1 = acc[tm][tn][4 * q + 1], x2 = acc[tm][tn][4 * q + 2],
                    x3 = acc[tm][tn][4 * q + 3];
        *reinterpret_cast<float4*>(s_out + row * E + col) =
            make_float4(rg_sigmoid(x0), rg_sigmoid(x1), rg_sigmoid(x2), rg_sigmoid(x3));
        if (logits_out) {  // 4-byte aligned only
          float* lo = logits_out + row * E + col;
          lo[0] = x0;
          lo[1] = x1;
          lo[2] = x2;
          lo[3] = x3;
        }
      }
  }
}

template <int E>
static int launch_rg(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, float* s_out,
                     float* logits_out, hipStream_t st) {
  const dim3 grid{unsigned((N + kRgBM - 1) / kRgBM), 1u, 1u};
  const dim3 block{unsigned(kRgThreads), 1u, 1u};
  hipLaunchKernelGGL((k_router_gemm<E, QB_RG_BK, QB_RG_STAGES>), grid, block, 0, st, hidden, w, N, H,
                     s_out, logits_out);
  return int(hipGetLastError());
}

int launch_router_gemm(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                       float* s_out, float* logits_out, hipStream_t st) {
  switch (E) {
    case 32: return launch_rg<32>(hidden, w, N, H, s_out, logits_out, st);
    case 64: return launch_rg<64>(hidden, w, N, H, s_out, logits_out, st);
    case 128: return launch_rg<128>(hidden, w, N, H, s_out, logits_out, st);
    case 256: return launch_rg<256>(hidden, w, N, H, s_out, logits_out, st);
    default: return int(hipErrorInvalidValue);
  }
}

}  // namespace qbk
