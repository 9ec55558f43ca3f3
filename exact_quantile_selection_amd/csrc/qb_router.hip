// qb_router.hip -- router GEMM on MFMA for the fused-router workload:
// logits[N][E] = hidden[N][H] . w[E][H]^T (bf16 inputs, fp32 accumulation),
// s = sigmoid(logits) written as the fp32 score matrix the balancing passes
// read.  The router's forward ("[Dev] Add global-batch quantile balancing",
// Megatron-LM PR #6637, Validation: real router forward/backward) produces
// the sigmoid scores of section "Quantile estimator".
//
// Tiling on gfx950: a workgroup of 4 waves owns 128 token rows and all E
// expert columns, so every token row is produced whole by one workgroup and
// `hidden` is read from HBM exactly once; the 2E*H-byte weight is re-read
// from L2.  Each wave computes 32 rows x E columns with E/32 accumulators of
// v_mfma_f32_32x32x16_bf16 (16 fp32 per lane each).  K advances in tiles of
// 64: the hidden tile [128][64] and weight tile [E][64] are staged in LDS
// (rows padded by 8 bf16 so the 16-byte operand reads of 32 consecutive rows
// fall in distinct banks), double-buffered, with the next tile's global
// loads in flight while the current one is multiplied.
//
// MFMA 32x32x16 bf16 operand layout (checked on the GPU): lane l supplies
// A[row = l % 32][k = 8 * (l / 32) + j] and B[k = 8 * (l / 32) + j][col = l % 32],
// j = 0..7; result element i of lane l is C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32].
#include <algorithm>

#include "qb_device.hpp"
#include "qb_internal.hpp"

namespace qbk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRgThreads = 256;
constexpr int kRgWaves = kRgThreads / kWave;
constexpr int kRgBM = 128;          // token rows per workgroup (32 per wave)
constexpr int kRgBK = 64;           // hidden dimension per K tile
constexpr int kRgLd = kRgBK + 8;    // padded LDS row length (bf16)

template <int E>
__global__ __launch_bounds__(kRgThreads) void k_router_gemm(const uint16_t* __restrict__ hidden,
                                                            const uint16_t* __restrict__ w,
                                                            int64_t N, int H,
                                                            float* __restrict__ s_out,
                                                            float* __restrict__ logits_out) {
  constexpr int T = E / 32;                         // accumulator tiles per wave
  constexpr int A_LOADS = kRgBM * kRgBK / 8 / kRgThreads;  // 16-byte loads per thread
  constexpr int B_LOADS = E * kRgBK / 8 / kRgThreads;
  __shared__ __align__(16) uint16_t lds_a[2][kRgBM * kRgLd];
  __shared__ __align__(16) uint16_t lds_b[2][E * kRgLd];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t m0 = int64_t(blockIdx.x) * kRgBM;
  const int KT = H / kRgBK;

  // Global -> register staging of one K tile (16-byte loads), and register
  // -> LDS stores.  Written out (no lambdas) so the staging registers stay
  // registers.
#define QB_RG_GLOAD(kt_)                                                                  \
  do {                                                                                    \
    const int k0_ = (kt_) * kRgBK;                                                        \
    _Pragma("unroll") for (int it = 0; it < A_LOADS; ++it) {                              \
      const int idx = it * kRgThreads + tid;                                              \
      const int row = idx / (kRgBK / 8), kc = idx % (kRgBK / 8);                          \
      int64_t gr = m0 + row;                                                              \
      gr = gr < N ? gr : N - 1;                                                           \
      ra[it] = *reinterpret_cast<const u32x4*>(hidden + gr * H + k0_ + kc * 8);           \
    }                                                                                     \
    _Pragma("unroll") for (int it = 0; it < B_LOADS; ++it) {                              \
      const int idx = it * kRgThreads + tid;                                              \
      const int e = idx / (kRgBK / 8), kc = idx % (kRgBK / 8);                            \
      rb[it] = *reinterpret_cast<const u32x4*>(w + int64_t(e) * H + k0_ + kc * 8);        \
    }                                                                                     \
  } while (0)
#define QB_RG_LSTORE(buf_)                                                                \
  do {                                                                                    \
    _Pragma("unroll") for (int it = 0; it < A_LOADS; ++it) {                              \
      const int idx = it * kRgThreads + tid;                                              \
      const int row = idx / (kRgBK / 8), kc = idx % (kRgBK / 8);                          \
      *reinterpret_cast<u32x4*>(&lds_a[(buf_)][row * kRgLd + kc * 8]) = ra[it];           \
    }                                                                                     \
    _Pragma("unroll") for (int it = 0; it < B_LOADS; ++it) {                              \
      const int idx = it * kRgThreads + tid;                                              \
      const int e = idx / (kRgBK / 8), kc = idx % (kRgBK / 8);                            \
      *reinterpret_cast<u32x4*>(&lds_b[(buf_)][e * kRgLd + kc * 8]) = rb[it];             \
    }                                                                                     \
  } while (0)

  u32x4 ra[A_LOADS], rb[B_LOADS];
  floatx16 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;

  QB_RG_GLOAD(0);
  QB_RG_LSTORE(0);
  __syncthreads();
  const int arow = wave * 32 + (lane % 32);
  const int kq = 8 * (lane / 32);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) QB_RG_GLOAD(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kRgBK / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&lds_a[buf][arow * kRgLd + ks * 16 + kq]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bf16x8 bv =
            *reinterpret_cast<const bf16x8*>(&lds_b[buf][(t * 32 + lane % 32) * kRgLd + ks * 16 + kq]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[t], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) QB_RG_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef QB_RG_GLOAD
#undef QB_RG_LSTORE

  // epilogue: sigmoid, store scores (and logits on request)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = m0 + wave * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
    if (row >= N) continue;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int col = t * 32 + (lane % 32);
      const float x = acc[t][i];
      s_out[row * E + col] = 1.0f / (1.0f + expf(-x));
      if (logits_out) logits_out[row * E + col] = x;
    }
  }
}

int launch_router_gemm(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                       float* s_out, float* logits_out, hipStream_t st) {
  const dim3 grid{unsigned((N + kRgBM - 1) / kRgBM), 1u, 1u};
  const dim3 block{unsigned(kRgThreads), 1u, 1u};
  switch (E) {
    case 32: hipLaunchKernelGGL(k_router_gemm<32>, grid, block, 0, st, hidden, w, N, H, s_out, logits_out); break;
    case 64: hipLaunchKernelGGL(k_router_gemm<64>, grid, block, 0, st, hidden, w, N, H, s_out, logits_out); break;
    case 128: hipLaunchKernelGGL(k_router_gemm<128>, grid, block, 0, st, hidden, w, N, H, s_out, logits_out); break;
    case 256: hipLaunchKernelGGL(k_router_gemm<256>, grid, block, 0, st, hidden, w, N, H, s_out, logits_out); break;
    default: return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace qbk
