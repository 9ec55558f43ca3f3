// qb_metrics.hip -- the load-balance metric MaxVio over expert loads.
//
// "Exact Quantile Balancing and Load-Error Injection for Mixture-of-Experts"
// (summary page): the background paragraph separates global balance (all
// tokens of an optimizer step) from local balance (inside each microbatch);
// the testbed paragraph defines MaxVio as how far the busiest expert of the
// worst layer exceeds the uniform share (a value of 5.96 is about 7x that
// share).  For a row of loads over n_tok tokens the uniform share is
// n_tok * K / E, and
//     v = fl32((double)max_e load_e / ((double)n_tok * K / E) - 1).
// Per layer the rows are its C microbatches (C = 1 for the global metric);
// the summary is [max over c, mean over c] (float64 sum in microbatch
// order), and `worst` the maximum of each over layers.
#include <climits>

#include "qb_device.hpp"
#include "qb_internal.hpp"

namespace qbk {

constexpr int kMvThreads = 256;

// One wave per row of E loads.
__global__ __launch_bounds__(kMvThreads) void k_maxvio_rows(const int32_t* __restrict__ load,
                                                            int64_t R, int E, int K, int64_t n_tok,
                                                            float* __restrict__ v) {
  const int64_t r = int64_t(blockIdx.x) * (kMvThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (r >= R) return;  // wave-uniform
  const int32_t* row = load + r * E;
  int m = INT_MIN;
  for (int e = lane; e < E; e += kWave) m = max(m, row[e]);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
  if (lane == 0) {
    const double share = double(n_tok) * double(K) / double(E);
    v[r] = float(double(m) / share - 1.0);
  }
}

// Per-layer summary and the worst layer; one workgroup.  Thread t owns
// layer l0 + t of a group of up to kMvThreads layers; the group's rows are
// staged through LDS in column chunks (all threads load, coalesced), and
// each thread then folds its own row in microbatch order (max, and the
// float64 sum).  Staged, the loads of a row are issued together instead
// of one dependent load per microbatch (8 -> ~2 us at 64 microbatches).
constexpr int kMvStage = 8192;  // staged floats (32 KiB)
__global__ __launch_bounds__(kMvThreads) void k_maxvio_summary(const float* __restrict__ v, int L,
                                                               int C, float* __restrict__ summary,
                                                               float* __restrict__ worst) {
  __shared__ float s_v[kMvStage];
  __shared__ float s_max[kMvThreads / kWave], s_mean[kMvThreads / kWave];
  const int t = threadIdx.x;
  float wmax = -__builtin_inff(), wmean = -__builtin_inff();
  for (int l0 = 0; l0 < L; l0 += kMvThreads) {
    const int nl = min(kMvThreads, L - l0);
    const int cc = kMvStage / nl - 1;  // columns per chunk; row stride cc + 1 (odd: no bank conflicts)
    float mx = __builtin_nanf("");     // fmaxf(NaN, x) = x: the fold starts at the row's first value
    double sum = 0.0;
    for (int c0 = 0; c0 < C; c0 += cc) {
      const int nc = min(cc, C - c0);
      __syncthreads();  // the previous chunk is consumed
      for (int i = t; i < nl * nc; i += kMvThreads) {
        const int li = i / nc, ci = i - li * nc;
        s_v[li * (cc + 1) + ci] = v[int64_t(l0 + li) * C + c0 + ci];
      }
      __syncthreads();
      if (t < nl) {
        const float* r = s_v + t * (cc + 1);
        for (int c = 0; c < nc; ++c) {
          mx = fmaxf(mx, r[c]);
          sum += double(r[c]);
        }
      }
    }
    if (t < nl) {
      const int l = l0 + t;
      const float mean = float(sum / double(C));
      if (summary) {
        summary[2 * l] = mx;
        summary[2 * l + 1] = mean;
      }
      wmax = fmaxf(wmax, mx);
      wmean = fmaxf(wmean, mean);
    }
  }
  // worst layer: wave maxima, then the waves' (maxima are exact in any order)
  const int lane = t & (kWave - 1);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    wmax = fmaxf(wmax, __shfl_xor(wmax, off));
    wmean = fmaxf(wmean, __shfl_xor(wmean, off));
  }
  if (lane == 0) {
    s_max[t / kWave] = wmax;
    s_mean[t / kWave] = wmean;
  }
  __syncthreads();
  if (t == 0 && worst) {
    float a = s_max[0], b = s_mean[0];
    for (int i = 1; i < kMvThreads / kWave; ++i) {
      a = fmaxf(a, s_max[i]);
      b = fmaxf(b, s_mean[i]);
    }
    worst[0] = a;
    worst[1] = b;
  }
}

// Small inputs (E <= 256, the rows fit kMvStage with a padded stride): the
// row values, the per-layer summary and the worst layer in one 1024-thread
// workgroup, the row values kept in LDS between the two; one launch instead
// of two.  Each wave takes four rows at a time and loads all of them before
// reducing any.  The same arithmetic in the same order as k_maxvio_rows +
// k_maxvio_summary (each layer's microbatches folded in order by one
// thread; the maxima are exact in any order), so the same values bit for
// bit.
constexpr int kMvSmallThreads = 1024;
__global__ __launch_bounds__(kMvSmallThreads) void k_maxvio_small(const int32_t* __restrict__ load, int L, int C,
                                                                  int E, int K, int64_t n_tok,
                                                                  float* __restrict__ v,
                                                                  float* __restrict__ summary,
                                                                  float* __restrict__ worst) {
  __shared__ float s_v[kMvStage];
  constexpr int kWaves = kMvSmallThreads / kWave;
  __shared__ float s_max[kWaves], s_mean[kWaves];
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int64_t R = int64_t(L) * C;
  const int stride = C + 1;  // padded row stride: consecutive layers start on different banks
  const double share = double(n_tok) * double(K) / double(E);
  for (int64_t r0 = wave; r0 < R; r0 += 4 * kWaves) {
    int m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t r = r0 + int64_t(k) * kWaves;
      int x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + q * kWave;
        x[q] = (r < R && e < E) ? load[r * E + e] : INT_MIN;
      }
      m[k] = max(max(x[0], x[1]), max(x[2], x[3]));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) m[k] = max(m[k], __shfl_xor(m[k], off));
      const int64_t r = r0 + int64_t(k) * kWaves;
      if (lane == 0 && r < R) {
        const float x = float(double(m[k]) / share - 1.0);
        v[r] = x;
        const int l = int(r / C), c = int(r - int64_t(l) * C);
        s_v[l * stride + c] = x;
      }
    }
  }
  __syncthreads();
  float wmax = -__builtin_inff(), wmean = -__builtin_inff();
  for (int l = t; l < L; l += kMvSmallThreads) {
    const float* r = s_v + l * stride;
    float mx = __builtin_nanf("");  // fmaxf(NaN, x) = x: the fold starts at the row's first value
    double sum = 0.0;
    for (int c = 0; c < C; ++c) {
      mx = fmaxf(mx, r[c]);
      sum += double(r[c]);
    }
    const float mean = float(sum / double(C));
    if (summary) {
      summary[2 * l] = mx;
      summary[2 * l + 1] = mean;
    }
    wmax = fmaxf(wmax, mx);
    wmean = fmaxf(wmean, mean);
  }
  // worst layer: wave maxima, then the waves' (maxima are exact in any order)
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    wmax = fmaxf(wmax, __shfl_xor(wmax, off));
    wmean = fmaxf(wmean, __shfl_xor(wmean, off));
  }
  if (lane == 0) {
    s_max[wave] = wmax;
    s_mean[wave] = wmean;
  }
  __syncthreads();
  if (t == 0 && worst) {
    float a = s_max[0], b = s_mean[0];
    for (int i = 1; i < kWaves; ++i) {
      a = fmaxf(a, s_max[i]);
      b = fmaxf(b, s_mean[i]);
    }
    worst[0] = a;
    worst[1] = b;
  }
}

int launch_maxvio(const int32_t* load, int L, int C, int E, int K, int64_t n_tok, float* v,
                  float* summary, float* worst, hipStream_t st) {
  const int64_t R = int64_t(L) * C;
  if ((summary || worst) && E <= 4 * kWave && int64_t(L) * (int64_t(C) + 1) <= kMvStage) {
    hipLaunchKernelGGL(k_maxvio_small, dim3(1u), dim3(kMvSmallThreads), 0, st, load, L, C, E, K, n_tok, v,
                       summary, worst);
    return int(hipGetLastError());
  }
  constexpr int kRowsPerBlock = kMvThreads / kWave;
  const dim3 grid{unsigned((R + kRowsPerBlock - 1) / kRowsPerBlock), 1u, 1u};
  const dim3 block{unsigned(kMvThreads), 1u, 1u};
  hipLaunchKernelGGL(k_maxvio_rows, grid, block, 0, st, load, R, E, K, n_tok, v);
  if (int rc = int(hipGetLastError())) return rc;
  if (summary || worst) {
    hipLaunchKernelGGL(k_maxvio_summary, dim3(1u), block, 0, st, v, L, C, summary, worst);
    return int(hipGetLastError());
  }
  return 0;
}

}  // namespace qbk
