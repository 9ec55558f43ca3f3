// qb_select.hip -- rank scans over the per-expert histograms and the bias
// update, one workgroup per layer.
//
// Method: "[Dev] Add global-batch quantile balancing" (Megatron-LM PR #6637):
// section "Quantile estimator" (b_next = K/E quantile of each expert's
// margins, then minus the mean; next range [min - 1, max + 1]), section
// "Implementation" (bias and bounds updated in place once), review thread
// (token total read from expert 0's row: every token adds one margin per
// expert).  "Exact Quantile Balancing and Load-Error Injection for
// Mixture-of-Experts" (summary page), EQB paragraph (find the bin holding the
// rank in the high-byte histogram, then the low byte inside it).
//
// Each wave scans one expert row at a time: lane l owns a contiguous block of
// ceil(n_bins/64) bins, the lane totals are prefix-summed across the wave
// (shuffles), a ballot finds the first lane whose running count reaches the
// rank, and that lane walks its block.  Everything that fixes floating-point
// rounding (the float64 mean, min/max) runs sequentially on one thread in
// expert order, so the result does not depend on the launch shape.
#include <algorithm>

#include "qb_device.hpp"
#include "qb_internal.hpp"
#include "../../include/qb.h"

namespace qbk {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxE = 256;

// Inclusive prefix sum of v over the wave.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

struct RankHit {
  int bin;         // first bin whose running count reaches the rank, -1 if none
  int64_t before;  // count of the bins below it
  int count;       // count of that bin
  int64_t total;   // row total
};

// Scan one histogram row for the first bin whose running count reaches
// `rank` (1-based).  All lanes of the wave return the same result.
__device__ RankHit scan_row(const int32_t* row, int n_bins, int64_t rank, int lane) {
  const int per = (n_bins + kWave - 1) / kWave;
  const int b0 = min(n_bins, lane * per);
  const int b1 = min(n_bins, b0 + per);
  int64_t mine = 0;
  for (int h = b0; h < b1; ++h) mine += row[h];
  const int64_t incl = wave_incl_scan(mine, lane);
  const int64_t excl = incl - mine;
  RankHit r;
  r.total = __shfl(incl, kWave - 1);
  const uint64_t hit = __ballot(incl >= rank && mine > 0);
  r.bin = -1;
  r.before = 0;
  r.count = 0;
  if (hit == 0) return r;
  const int f = __ffsll((unsigned long long)hit) - 1;
  int bin = -1;
  int64_t before = 0;
  int cnt = 0;
  if (lane == f) {
    int64_t run = excl;
    for (int h = b0; h < b1; ++h) {
      const int c = row[h];
      if (run + c >= rank) {
        bin = h;
        before = run;
        cnt = c;
        break;
      }
      run += c;
    }
  }
  r.bin = __shfl(bin, f);
  r.before = __shfl(before, f);
  r.count = __shfl(cnt, f);
  return r;
}

__global__ __launch_bounds__(kSelThreads) void k_select(
    int phase, int E, int K, const int32_t* __restrict__ hist, int n_bins,
    int32_t* __restrict__ sel_hi, int32_t* __restrict__ rank_lo, uint16_t* __restrict__ key_out,
    float* __restrict__ q_out, float* __restrict__ b, float* __restrict__ bounds,
    int32_t* __restrict__ err) {
  __shared__ int64_t s_total;
  __shared__ int s_err;
  __shared__ float s_q[kMaxE];
  __shared__ float s_bn[kMaxE];
  __shared__ double s_mean;
  __shared__ float s_lohi[2];
  const int layer = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nb = phase == QB_SELECT_UNIFORM ? n_bins : 256;
  hist += int64_t(layer) * E * nb;
  const int64_t le = int64_t(layer) * E;

  if (wave == 0) {
    int64_t t = 0;
    for (int h = lane; h < nb; h += kWave) t += hist[h];
    t = wave_incl_scan(t, lane);
    if (lane == kWave - 1) s_total = t;
  }
  if (tid == 0) {
    s_err = 0;
    s_lohi[0] = 0.0f;
    s_lohi[1] = 1.0f;
    if (phase == QB_SELECT_UNIFORM) {
      s_lohi[0] = bounds[2 * layer];
      s_lohi[1] = bounds[2 * layer + 1];
    }
  }
  __syncthreads();
  const int64_t total = s_total;
  const int64_t m = (int64_t(K) * total + E - 1) / E;  // 1-based rank ceil(K*N/E)
  if (tid == 0 && total == 0 && phase != QB_SELECT_LO) atomicOr(&s_err, QB_ERR_EMPTY);
  const double lo = double(s_lohi[0]);
  const double w = (double(s_lohi[1]) - lo) / double(n_bins);

  for (int j = wave; j < E; j += kSelWaves) {
    const int32_t* row = hist + int64_t(j) * nb;
    int64_t rank = m;
    int hi_byte = 0;
    if (phase == QB_SELECT_LO) {
      hi_byte = sel_hi[le + j];
      rank = rank_lo[le + j];
      if (hi_byte < 0 || hi_byte > 255 || rank < 1) {
        if (lane == 0) atomicOr(&s_err, QB_ERR_RANK);
        continue;
      }
    }
    const RankHit h = scan_row(row, nb, rank, lane);
    if (lane != 0) continue;
    if (phase != QB_SELECT_LO && h.total != total) atomicOr(&s_err, QB_ERR_ROW_TOTALS);
    if (h.bin < 0) {
      atomicOr(&s_err, QB_ERR_RANK);
      if (phase == QB_SELECT_HI) {
        sel_hi[le + j] = -1;
        rank_lo[le + j] = 0;
      }
      continue;
    }
    if (phase == QB_SELECT_HI) {
      sel_hi[le + j] = h.bin;
      rank_lo[le + j] = int32_t(rank - h.before);
    } else if (phase == QB_SELECT_LO) {
      const uint32_t key = (uint32_t(hi_byte) << 8) | uint32_t(h.bin);
      s_q[j] = __builtin_bit_cast(float, unkey16(key) << 16);
      if (key_out) key_out[le + j] = uint16_t(key);
    } else {
      const double frac = double(rank - h.before) / double(h.count);
      s_q[j] = float(lo + w * (double(h.bin) + frac));
    }
  }
  __syncthreads();
  if (phase == QB_SELECT_HI || s_err != 0) {
    if (tid == 0 && s_err && err) atomicOr(err, s_err);
    return;
  }
  // b_next = q - mean(q): float64 sum in expert order, one rounding to fp32.
  if (tid == 0) {
    double sum = 0.0;
    for (int j = 0; j < E; ++j) sum += double(s_q[j]);
    s_mean = sum / double(E);
  }
  __syncthreads();
  for (int j = tid; j < E; j += kSelThreads) {
    const float bn = float(double(s_q[j]) - s_mean);
    s_bn[j] = bn;
    b[le + j] = bn;
    if (q_out) q_out[le + j] = s_q[j];
  }
  __syncthreads();
  if (tid == 0) {
    float mn = s_bn[0], mx = s_bn[0];
    for (int j = 1; j < E; ++j) {
      if (s_bn[j] < mn) mn = s_bn[j];
      if (s_bn[j] > mx) mx = s_bn[j];
    }
    bounds[2 * layer] = mn - 1.0f;
    bounds[2 * layer + 1] = mx + 1.0f;
  }
}

int launch_select(int phase, int L, int E, int K, const int32_t* hist, int n_bins,
                  int32_t* sel_hi, int32_t* rank_lo, uint16_t* key_out, float* q_out, float* b,
                  float* bounds, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(unsigned(L)), dim3(kSelThreads), 0, st, phase, E, K, hist,
                     n_bins, sel_hi, rank_lo, key_out, q_out, b, bounds, err);
  return int(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Next-range seed for the K3 mode: bounds = [min b - 1, max b + 1].
__global__ void k_bias_bounds(const float* __restrict__ b, int L, int E, float* __restrict__ bounds) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= L) return;
  const float* bl = b + int64_t(l) * E;
  float mn = bl[0], mx = bl[0];
  for (int j = 1; j < E; ++j) {
    if (bl[j] < mn) mn = bl[j];
    if (bl[j] > mx) mx = bl[j];
  }
  bounds[2 * l] = mn - 1.0f;
  bounds[2 * l + 1] = mx + 1.0f;
}

int launch_bias_bounds(const float* b, int L, int E, float* bounds, hipStream_t st) {
  hipLaunchKernelGGL(k_bias_bounds, dim3(unsigned((L + 63) / 64)), dim3(64), 0, st, b, L, E, bounds);
  return int(hipGetLastError());
}

// ---------------------------------------------------------------------------
__global__ void k_fill_i32(int32_t* __restrict__ dst, int64_t count, int32_t value) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const uintptr_t mis = (reinterpret_cast<uintptr_t>(dst) & 15u) / 4u;
  const int64_t head = mis ? min(count, int64_t(4 - mis)) : 0;
  for (int64_t i = i0; i < head; i += stride) dst[i] = value;
  int4* d4 = reinterpret_cast<int4*>(dst + head);
  const int64_t n4 = (count - head) / 4;
  const int4 v4 = make_int4(value, value, value, value);
  for (int64_t i = i0; i < n4; i += stride) d4[i] = v4;
  for (int64_t i = head + n4 * 4 + i0; i < count; i += stride) dst[i] = value;
}

int launch_fill_i32(int32_t* dst, int64_t count, int32_t value, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>(2048, (count / 4 + 255) / 256 + 1);
  hipLaunchKernelGGL(k_fill_i32, dim3(unsigned(blocks)), dim3(256), 0, st, dst, count, value);
  return int(hipGetLastError());
}

}  // namespace qbk
