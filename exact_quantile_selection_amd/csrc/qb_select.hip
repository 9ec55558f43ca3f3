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
// The rank scans run one wave per expert row (E/16 workgroups per layer):
// lane l owns a contiguous block of ceil(n_bins/64) bins, the lane totals
// are prefix-summed across the wave (shuffles), a ballot finds the first
// lane whose running count reaches the rank, and that lane walks its block.
// The workspace selects (low byte, K3) first sum the passes' per-workgroup
// partial rows, one workgroup per expert, then scan the sum.  A small
// per-layer kernel then forms the bias update; the float64 mean runs
// sequentially on one thread in expert order, so the result does not
// depend on the launch shape.
#include <algorithm>

#include "qb_device.hpp"
#include "qb_internal.hpp"
#include "../../include/qb.h"

namespace qbk {

#ifndef QB_SEL_WAVES
#define QB_SEL_WAVES 16
#endif
constexpr int kRowWaves = QB_SEL_WAVES;         // experts per workgroup (one per wave)
constexpr int kRowThreads = kRowWaves * kWave;
constexpr int kFinThreads = 256;                // >= E: one thread per expert

// Inclusive prefix sum of v over the wave.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

// PER consecutive bins of a row owned by this lane (zero past n_bins); the
// 64 lanes of the wave read the row contiguously.
template <int PER>
__device__ __forceinline__ void load_bins(const int32_t* row, int n_bins, bool vec, int lane,
                                          int (&c)[PER]) {
  const int b0 = lane * PER;
  if (vec && b0 + PER <= n_bins) {
#pragma unroll
    for (int k = 0; k < PER; k += 4) {
      const int4 v = *reinterpret_cast<const int4*>(row + b0 + k);
      c[k] = v.x;
      c[k + 1] = v.y;
      c[k + 2] = v.z;
      c[k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) c[k] = (b0 + k < n_bins) ? row[b0 + k] : 0;
  }
}

// Per-expert rank scans, one wave per expert row, E/16 workgroups per layer.
//   HI: sel_hi / rank_lo from the high-byte histogram.
//   LO: key (sel_hi << 8 | low byte) and its bf16 value into q_out.
//   UNIFORM: in-bin linear interpolation into q_out.
// A failed row writes sel_hi = -1 (HI) or q = NaN (LO, UNIFORM), which the
// finalize kernel turns into "layer left unchanged".
template <int PER>
__global__ __launch_bounds__(kRowThreads) void k_select_rows(
    int phase, int E, int K, const int32_t* __restrict__ hist, int n_bins, int vec,
    int32_t* __restrict__ sel_hi, int32_t* __restrict__ rank_lo, uint16_t* __restrict__ key_out,
    float* __restrict__ q_out, const float* __restrict__ bounds, int32_t* __restrict__ err) {
  const int layer = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = blockIdx.x * kRowWaves + int(threadIdx.x / kWave);
  if (j >= E) return;  // whole wave; no workgroup barrier follows
  const int64_t le = int64_t(layer) * E;
  const int32_t* lh = hist + le * n_bins;

  int64_t rank;
  int hi_byte = 0;
  int bits = 0;
  if (phase == QB_SELECT_LO) {
    hi_byte = sel_hi[le + j];
    rank = rank_lo[le + j];
  }
  int c[PER];
  load_bins<PER>(lh + int64_t(j) * n_bins, n_bins, vec != 0, lane, c);
  int64_t mine = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) mine += c[k];
  if (phase == QB_SELECT_LO) {
    if (hi_byte < 0 || hi_byte > 255 || rank < 1) {
      if (lane == 0) {
        q_out[le + j] = __builtin_nanf("");
        if (err) atomicOr(err, QB_ERR_RANK);
      }
      return;
    }
  } else {
    // token total from expert 0's row (each token adds one margin per expert)
    int c0[PER];
    load_bins<PER>(lh, n_bins, vec != 0, lane, c0);
    int64_t t0 = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) t0 += c0[k];
    const int64_t total = wave_sum(t0);
    if (total == 0) bits |= QB_ERR_EMPTY;
    if (wave_sum(mine) != total) bits |= QB_ERR_ROW_TOTALS;
    rank = (int64_t(K) * total + E - 1) / E;  // 1-based rank ceil(K*N/E)
  }

  const int64_t incl = wave_incl_scan(mine, lane);
  const uint64_t hit = __ballot(incl >= rank && mine > 0);
  int bin = -1, cnt = 0;
  int64_t before = 0;
  if (hit != 0) {
    const int f = __ffsll((unsigned long long)hit) - 1;
    if (lane == f) {
      int64_t run = incl - mine;
      bool found = false;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        if (!found && run + c[k] >= rank) {
          found = true;
          bin = lane * PER + k;
          before = run;
          cnt = c[k];
        }
        if (!found) run += c[k];
      }
    }
    bin = __shfl(bin, f);
    before = __shfl(before, f);
    cnt = __shfl(cnt, f);
  }
  if (lane != 0) return;
  if (bin < 0) bits |= QB_ERR_RANK;
  if (bits && err) atomicOr(err, bits);
  if (phase == QB_SELECT_HI) {
    sel_hi[le + j] = bin < 0 ? -1 : bin;
    rank_lo[le + j] = bin < 0 ? 0 : int32_t(rank - before);
  } else if (phase == QB_SELECT_LO) {
    if (bin < 0) {
      q_out[le + j] = __builtin_nanf("");
      return;
    }
    const uint32_t key = (uint32_t(hi_byte) << 8) | uint32_t(bin);
    q_out[le + j] = __builtin_bit_cast(float, unkey16(key) << 16);
    if (key_out) key_out[le + j] = uint16_t(key);
  } else {
    if (bin < 0 || bits) {
      q_out[le + j] = __builtin_nanf("");
      return;
    }
    const double lo = double(bounds[2 * layer]);
    const double w = (double(bounds[2 * layer + 1]) - lo) / double(n_bins);
    const double frac = double(rank - before) / double(cnt);
    q_out[le + j] = float(lo + w * (double(bin) + frac));
  }
}

// Rank scan over a full 16-bit key histogram ([L][E][65536]): one
// workgroup per (expert, layer); thread t owns bins [256 t, 256 t + 256).
// The rank is ceil(K * T / E) with T the row's own total (every row of a
// valid histogram holds one key per token); the bin holding it is the key.
constexpr int kFullThreads = 256;
__global__ __launch_bounds__(kFullThreads) void k_select_full(int E, int K, const int32_t* __restrict__ hist,
                                                              uint16_t* __restrict__ key_out,
                                                              float* __restrict__ q_out,
                                                              int32_t* __restrict__ err) {
  constexpr int PER = 65536 / kFullThreads;
  __shared__ int64_t s_incl[kFullThreads];
  __shared__ int s_owner;
  const int j = blockIdx.x, layer = blockIdx.y, tid = threadIdx.x;
  const int64_t le = int64_t(layer) * E;
  const int32_t* row = hist + (le + j) * 65536 + int64_t(tid) * PER;
  int64_t mine = 0;
#pragma unroll 8
  for (int k = 0; k < PER; k += 4) {
    const int4 v = *reinterpret_cast<const int4*>(row + k);
    mine += int64_t(v.x) + v.y + v.z + v.w;
  }
  s_incl[tid] = mine;
  if (tid == 0) s_owner = -1;
  __syncthreads();
  // inclusive prefix over the 256 thread totals (Hillis-Steele in LDS)
  for (int d = 1; d < kFullThreads; d <<= 1) {
    const int64_t o = tid >= d ? s_incl[tid - d] : 0;
    __syncthreads();
    s_incl[tid] += o;
    __syncthreads();
  }
  const int64_t total = s_incl[kFullThreads - 1];
  const int64_t rank = (int64_t(K) * total + E - 1) / E;
  const int64_t incl = s_incl[tid];
  const int64_t excl = incl - mine;
  if (rank >= 1 && excl < rank && incl >= rank) s_owner = tid;  // exactly one thread
  __syncthreads();
  if (tid != s_owner) {
    if (tid == 0 && s_owner < 0) {
      q_out[le + j] = __builtin_nanf("");
      if (err) atomicOr(err, total == 0 ? QB_ERR_EMPTY : QB_ERR_RANK);
    }
    return;
  }
  int64_t run = excl;
  int bin = -1;
  for (int k = 0; k < PER; ++k) {
    run += row[k];
    if (run >= rank) {
      bin = tid * PER + k;
      break;
    }
  }
  const uint32_t key = uint32_t(bin);
  q_out[le + j] = __builtin_bit_cast(float, unkey16(key) << 16);
  if (key_out) key_out[le + j] = uint16_t(key);
}

// The float64 sum of the q values is exact, and so equal in every order,
// when all of its partial sums fit 53 bits: every term is a multiple of
// 2^lo (lo: the exponent of the lowest set bit of the term with the lowest
// one) and the sum of at most 256 terms below 2^hi in magnitude stays below
// 2^(hi + 8).  Then a tree reduction gives the sum of the expert-order loop
// bit for bit (zeros enter as +0, as the loop's 0.0 start makes them); a
// wider spread keeps the loop (1).  The loop alone: 0.
#ifndef QB_FIN_TREE
#define QB_FIN_TREE 1
#endif

// Exponents bounding a finite fp32 value v != 0: v is a multiple of 2^lo
// and |v| < 2^hi.
__device__ __forceinline__ void exp_span(float v, int& lo, int& hi) {
  const uint32_t u = __float_as_uint(v);
  const int ex = int((u >> 23) & 0xFFu);
  const uint32_t m = ex ? ((u & 0x7FFFFFu) | 0x800000u) : (u & 0x7FFFFFu);
  lo = (ex ? ex - 150 : -149) + __builtin_ctz(m);
  hi = ex ? ex - 126 : -126;
}

// b_next = q - mean(q) (the float64 sum of q in expert order, one rounding
// to fp32), written over b; bounds = [min - 1, max + 1] (min and
// max as a parallel reduction: any order gives the same values up to the
// sign of a zero, which the -1 / +1 removes).  A layer with a NaN quantile
// (failed rank search) keeps its b and bounds.  Run by the first
// kFinThreads threads of a workgroup for one layer (q, b: that layer's E
// entries; bounds: its pair); every thread of the workgroup calls it.
__device__ void finalize_layer(int E, const float* q, float* b, float* bounds, int32_t* err, int tid) {
  __shared__ __align__(16) float sq[kFinThreads];
  __shared__ double s_mean;
  __shared__ int s_bad;
  __shared__ float s_min[kFinThreads / kWave], s_max[kFinThreads / kWave];
  __shared__ double s_sum[kFinThreads / kWave];
  __shared__ int s_lo[kFinThreads / kWave], s_hi[kFinThreads / kWave];
  const int lane = tid & (kWave - 1);
  const bool mine = tid < kFinThreads;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < E) {
    const float v = q[tid];
    sq[tid] = v;
    if (v != v) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0 && err) atomicOr(err, QB_ERR_RANK);
    return;
  }
  bool tree = false;
  if constexpr (QB_FIN_TREE != 0) {
    const int lane_ = tid & (kWave - 1);
    int lo = 1 << 20, hi = -(1 << 20);
    double d = 0.0;
    if (tid < E) {
      const float v = sq[tid];
      if (v != 0.0f) exp_span(v, lo, hi);
      d = double(v) + 0.0;
    }
#pragma unroll
    for (int k = 1; k < kWave; k <<= 1) {
      lo = min(lo, __shfl_xor(lo, k));
      hi = max(hi, __shfl_xor(hi, k));
      d += __shfl_xor(d, k);
    }
    if (mine && lane_ == 0) {
      s_lo[tid / kWave] = lo;
      s_hi[tid / kWave] = hi;
      s_sum[tid / kWave] = d;
    }
    __syncthreads();
    lo = s_lo[0];
    hi = s_hi[0];
#pragma unroll
    for (int w = 1; w < kFinThreads / kWave; ++w) {
      lo = min(lo, s_lo[w]);
      hi = max(hi, s_hi[w]);
    }
    tree = hi + 8 - lo <= 53;  // also true when every q is zero
    if (tree && tid == 0) {
      double sum = s_sum[0];
      for (int w = 1; w < kFinThreads / kWave; ++w) sum += s_sum[w];
      s_mean = sum / double(E);
    }
  }
  if (!tree && tid == 0) {
    // E is a multiple of 4; vector LDS reads keep the in-order float64 chain
    // from waiting on one LDS round trip per term.
    double sum = 0.0;
    const float4* q4 = reinterpret_cast<const float4*>(sq);
#pragma unroll 8
    for (int k = 0; k < E / 4; ++k) {
      const float4 v = q4[k];
      sum += double(v.x);
      sum += double(v.y);
      sum += double(v.z);
      sum += double(v.w);
    }
    s_mean = sum / double(E);
  }
  __syncthreads();
  float mn = __builtin_inff(), mx = -__builtin_inff();
  if (tid < E) {
    const float bn = float(double(sq[tid]) - s_mean);
    b[tid] = bn;
    mn = bn;
    mx = bn;
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, d));
    mx = fmaxf(mx, __shfl_xor(mx, d));
  }
  if (mine && lane == 0) {
    s_min[tid / kWave] = mn;
    s_max[tid / kWave] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kFinThreads / kWave; ++w) {
      mn = fminf(mn, s_min[w]);
      mx = fmaxf(mx, s_max[w]);
    }
    bounds[0] = mn - 1.0f;
    bounds[1] = mx + 1.0f;
  }
}

// One workgroup per layer.
__global__ __launch_bounds__(kFinThreads) void k_finalize(int E, const float* __restrict__ q,
                                                          float* __restrict__ b,
                                                          float* __restrict__ bounds,
                                                          int32_t* __restrict__ err) {
  const int layer = blockIdx.x;
  const int64_t le = int64_t(layer) * E;
  finalize_layer(E, q + le, b + le, bounds + 2 * layer, err, threadIdx.x);
}

// Low-byte select from per-workgroup partial histograms (the workspace of
// qb_radix_hist_lo_ws): one workgroup per (expert, layer).  Expert j's G
// partial rows are contiguous (G x 256 bytes, or G x 512 for the rows
// stored as uint16, picked by the row flags); 32 lanes read one row with
// 8-byte (16-byte) loads of 8 bins each, so the workgroup reads kLoWsRows
// rows per trip.  The per-thread sums meet in LDS and thread h adds bin h over the
// row groups: integer sums, so the counts equal those of the atomic path.
// The summed row optionally goes to hist_lo; then the first bin whose
// running count reaches rank_lo is the low byte.
constexpr int kLoWsThreads = 1024;
constexpr int kLoWsRows = kLoWsThreads / 32;
__global__ __launch_bounds__(kLoWsThreads) void k_select_lo_ws(int E, int G, const uint8_t* __restrict__ ws,
                                                               int64_t ws_flag, int64_t ws_p16,
                                                               const int32_t* __restrict__ sel_hi,
                                                               const int32_t* __restrict__ rank_lo,
                                                               int32_t* __restrict__ hist_lo,
                                                               uint16_t* __restrict__ key_out,
                                                               float* __restrict__ q_out,
                                                               int32_t* __restrict__ hist_hi,
                                                               int32_t* __restrict__ err) {
  __shared__ __align__(16) int32_t s_part[kLoWsRows][256];
  __shared__ int64_t s_wave[256 / kWave];
  __shared__ int s_bin;
  const int j = blockIdx.x, layer = blockIdx.y, t = threadIdx.x;
  const int64_t le = int64_t(layer) * E;
  const int c8 = t & 31, r0 = t >> 5;
  // Partial row g of expert j: bytes at p8[32 g] (8 per thread) unless
  // its flag says uint16, then p16[32 g] (8 uint16 per thread).
  const int64_t row0 = (le + j) * G;
  const uint8_t* flag = ws + ws_flag + row0;
  const uint2* p8 = reinterpret_cast<const uint2*>(ws + row0 * 256) + c8;
  const uint4* p16 = reinterpret_cast<const uint4*>(ws + ws_p16 + row0 * 512) + c8;
  int32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add8 = [&](const uint2& v) {
    acc[0] += int32_t(v.x & 0xFFu);
    acc[1] += int32_t((v.x >> 8) & 0xFFu);
    acc[2] += int32_t((v.x >> 16) & 0xFFu);
    acc[3] += int32_t(v.x >> 24);
    acc[4] += int32_t(v.y & 0xFFu);
    acc[5] += int32_t((v.y >> 8) & 0xFFu);
    acc[6] += int32_t((v.y >> 16) & 0xFFu);
    acc[7] += int32_t(v.y >> 24);
  };
  auto add16 = [&](const uint4& v) {
    acc[0] += int32_t(v.x & 0xFFFFu);
    acc[1] += int32_t(v.x >> 16);
    acc[2] += int32_t(v.y & 0xFFFFu);
    acc[3] += int32_t(v.y >> 16);
    acc[4] += int32_t(v.z & 0xFFFFu);
    acc[5] += int32_t(v.z >> 16);
    acc[6] += int32_t(v.w & 0xFFFFu);
    acc[7] += int32_t(v.w >> 16);
  };
  auto add_row = [&](int gg, const uint2& v8, uint8_t f) {
    if (f)
      add16(p16[int64_t(gg) * 32]);
    else
      add8(v8);
  };
  int g = r0;
  for (; g + 3 * kLoWsRows < G; g += 4 * kLoWsRows) {
    const uint8_t f0 = flag[g], f1 = flag[g + kLoWsRows], f2 = flag[g + 2 * kLoWsRows],
                  f3 = flag[g + 3 * kLoWsRows];
    const uint2 v0 = p8[int64_t(g) * 32];
    const uint2 v1 = p8[int64_t(g + kLoWsRows) * 32];
    const uint2 v2 = p8[int64_t(g + 2 * kLoWsRows) * 32];
    const uint2 v3 = p8[int64_t(g + 3 * kLoWsRows) * 32];
    add_row(g, v0, f0);
    add_row(g + kLoWsRows, v1, f1);
    add_row(g + 2 * kLoWsRows, v2, f2);
    add_row(g + 3 * kLoWsRows, v3, f3);
  }
  for (; g < G; g += kLoWsRows) add_row(g, p8[int64_t(g) * 32], flag[g]);
  int4* dst = reinterpret_cast<int4*>(&s_part[r0][8 * c8]);
  dst[0] = make_int4(acc[0], acc[1], acc[2], acc[3]);
  dst[1] = make_int4(acc[4], acc[5], acc[6], acc[7]);
  if (t == 0) s_bin = -1;
  __syncthreads();
  // Threads 0..255 (waves 0..3) own one bin each from here on; the other
  // waves only meet the barriers.
  const int h = t;
  const int lane = t & (kWave - 1), wave = t / kWave;
  int32_t c = 0;
  int64_t incl = 0;
  if (h < 256) {
#pragma unroll 8
    for (int r = 0; r < kLoWsRows; ++r) c += s_part[r][h];
    if (hist_lo) hist_lo[(le + j) * 256 + h] = c;
    // inclusive prefix over the 256 bins: wave scans, then wave offsets
    incl = wave_incl_scan(int64_t(c), lane);
    if (lane == kWave - 1) s_wave[wave] = incl;
  }
  __syncthreads();
  const int hi_byte = sel_hi[le + j];
  const int64_t rank = rank_lo[le + j];
  const bool ok = hi_byte >= 0 && hi_byte <= 255 && rank >= 1;
  if (h < 256) {
    for (int w = 0; w < wave; ++w) incl += s_wave[w];
    if (ok && c > 0 && incl >= rank && incl - c < rank) s_bin = h;  // exactly one bin
  }
  // The high-byte histogram of this update has been read (select HI ran
  // before pass 2): clear expert j's row in place for the next update.
  if (hist_hi && h < 256) hist_hi[(le + j) * 256 + h] = 0;
  __syncthreads();
  if (h != 0) return;
  const int bin = s_bin;
  if (!ok || bin < 0) {
    q_out[le + j] = __builtin_nanf("");
    if (err) atomicOr(err, QB_ERR_RANK);
    return;
  }
  const uint32_t key = (uint32_t(hi_byte) << 8) | uint32_t(bin);
  q_out[le + j] = __builtin_bit_cast(float, unkey16(key) << 16);
  if (key_out) key_out[le + j] = uint16_t(key);
}

int launch_select(int phase, int L, int E, int K, const int32_t* hist, int n_bins,
                  int32_t* sel_hi, int32_t* rank_lo, uint16_t* key_out, float* q_out, float* b,
                  float* bounds, int32_t* err, hipStream_t st) {
  if (phase == QB_SELECT_FULL) {
    hipLaunchKernelGGL(k_select_full, dim3(unsigned(E), unsigned(L)), dim3(kFullThreads), 0, st, E, K, hist,
                       key_out, q_out, err);
    if (int rc = int(hipGetLastError())) return rc;
    hipLaunchKernelGGL(k_finalize, dim3(unsigned(L)), dim3(kFinThreads), 0, st, E, q_out, b, bounds, err);
    return int(hipGetLastError());
  }
  const int vec = ((n_bins % 4) == 0 && (reinterpret_cast<uintptr_t>(hist) & 15u) == 0) ? 1 : 0;
  const dim3 grid{unsigned((E + kRowWaves - 1) / kRowWaves), unsigned(L), 1u};
  const dim3 block{unsigned(kRowThreads), 1u, 1u};
  if (n_bins <= 256)
    hipLaunchKernelGGL(k_select_rows<4>, grid, block, 0, st, phase, E, K, hist, n_bins, vec, sel_hi,
                       rank_lo, key_out, q_out, bounds, err);
  else if (n_bins <= 1024)
    hipLaunchKernelGGL(k_select_rows<16>, grid, block, 0, st, phase, E, K, hist, n_bins, vec, sel_hi,
                       rank_lo, key_out, q_out, bounds, err);
  else
    hipLaunchKernelGGL(k_select_rows<32>, grid, block, 0, st, phase, E, K, hist, n_bins, vec, sel_hi,
                       rank_lo, key_out, q_out, bounds, err);
  int rc = int(hipGetLastError());
  if (rc != int(hipSuccess) || phase == QB_SELECT_HI) return rc;
  hipLaunchKernelGGL(k_finalize, dim3(unsigned(L)), dim3(kFinThreads), 0, st, E, q_out, b, bounds, err);
  return int(hipGetLastError());
}

int launch_select_lo_ws(int L, int E, int G, const uint8_t* ws, const int32_t* sel_hi, const int32_t* rank_lo,
                        int32_t* hist_lo, uint16_t* key_out, float* q_out, float* b, float* bounds,
                        int32_t* hist_hi, int32_t* err, hipStream_t st) {
  const LoWs lay = lo_ws_layout(L, E, G);
  hipLaunchKernelGGL(k_select_lo_ws, dim3(unsigned(E), unsigned(L)), dim3(kLoWsThreads), 0, st, E, G, ws, lay.flag,
                     lay.p16, sel_hi, rank_lo, hist_lo, key_out, q_out, hist_hi, err);
  if (int rc = int(hipGetLastError())) return rc;
  hipLaunchKernelGGL(k_finalize, dim3(unsigned(L)), dim3(kFinThreads), 0, st, E, q_out, b, bounds, err);
  return int(hipGetLastError());
}

// K3 select from the binning pass's partial rows (qb_uniform_hist_ws): one
// 1024-thread workgroup per (expert, layer).  Thread t adds bins
// 8 (t % 128) .. + 7 (and + 1024 on a second step for more than 1024 bins)
// over the rows t / 128, t / 128 + 8, ... of its expert, one 16-byte
// (uint16 row) or 8-byte (byte row) load per row, with the rows' flags
// staged in LDS first so that no load waits for its flag; the eight row
// groups meet in LDS.  Then threads 0..255 each own a contiguous run of the
// summed bins, and the rank scan and the in-bin interpolation are those of
// k_select_rows (UNIFORM), with the token count N given (every token adds
// one margin per expert, so every consistent row sums to N).  The summed row
// optionally goes to hist_u (overwritten).
constexpr int kUWsThreads = 1024;
constexpr int kUWsGroups = kUWsThreads / 128;  // row groups
__global__ __launch_bounds__(kUWsThreads) void k_select_uniform_ws(int64_t N, int E, int K, int n_bins, int G,
                                                                   const uint8_t* __restrict__ ws, UhWs wl,
                                                                   int32_t* __restrict__ hist_u,
                                                                   float* __restrict__ q_out,
                                                                   const float* __restrict__ bounds,
                                                                   int32_t* __restrict__ err) {
  __shared__ __align__(16) int32_t s_part[kUWsGroups][2048];
  __shared__ uint8_t s_flag[kUWsThreads];
  __shared__ int64_t s_wave[256 / kWave];
  __shared__ int s_bin;
  __shared__ int64_t s_before;
  __shared__ int32_t s_cnt;
  const int j = blockIdx.x, layer = blockIdx.y, t = threadIdx.x;
  const int c8 = t & 127, rg = t >> 7;
  const int64_t row0 = (int64_t(layer) * E + j) * G;
  int32_t acc[2][8] = {};  // bins 8 c8 + k, and + 1024
  for (int g0 = 0; g0 < G; g0 += kUWsThreads) {
    const int gn = G - g0 < kUWsThreads ? G - g0 : kUWsThreads;
    __syncthreads();  // the previous chunk's flags are read
    if (t < gn) s_flag[t] = ws[wl.flag + row0 + g0 + t];
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int b = 8 * c8 + 1024 * pass;
      if (b >= n_bins) break;
#pragma unroll 8
      for (int gi = rg; gi < gn; gi += kUWsGroups) {
        const int64_t r = row0 + g0 + gi;
        if (s_flag[gi]) {
          const uint4 v = *reinterpret_cast<const uint4*>(ws + wl.p16 + r * wl.b16 + 2 * b);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[pass][2 * k] += int32_t(w[k] & 0xFFFFu);
            acc[pass][2 * k + 1] += int32_t(w[k] >> 16);
          }
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(ws + wl.p8 + r * wl.b8 + b);
          const uint32_t w[2] = {v.x, v.y};
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            acc[pass][4 * k] += int32_t(w[k] & 0xFFu);
            acc[pass][4 * k + 1] += int32_t((w[k] >> 8) & 0xFFu);
            acc[pass][4 * k + 2] += int32_t((w[k] >> 16) & 0xFFu);
            acc[pass][4 * k + 3] += int32_t(w[k] >> 24);
          }
        }
      }
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int b = 8 * c8 + 1024 * pass;
    if (b < n_bins) {
      int4* dst = reinterpret_cast<int4*>(&s_part[rg][b]);
      dst[0] = make_int4(acc[pass][0], acc[pass][1], acc[pass][2], acc[pass][3]);
      dst[1] = make_int4(acc[pass][4], acc[pass][5], acc[pass][6], acc[pass][7]);
    }
  }
  if (t == 0) s_bin = -1;
  __syncthreads();
  const int per = (n_bins + 255) / 256;  // <= 8
  const int lane = t & (kWave - 1), wave = t / kWave;
  const int h0 = t * per;
  auto summed = [&](int h) {
    int32_t c = 0;
#pragma unroll
    for (int q = 0; q < kUWsGroups; ++q) c += s_part[q][h];
    return c;
  };
  int64_t mine = 0, incl = 0;
  if (t < 256) {
    for (int k = 0; k < per; ++k) {
      const int h = h0 + k;
      if (h < n_bins) {
        const int32_t c = summed(h);
        mine += c;
        if (hist_u) hist_u[(int64_t(layer) * E + j) * n_bins + h] = c;
      }
    }
    incl = wave_incl_scan(mine, lane);
    if (lane == kWave - 1) s_wave[wave] = incl;
  }
  __syncthreads();
  const int64_t rank = (int64_t(K) * N + E - 1) / E;  // 1-based rank ceil(K*N/E)
  int64_t total = 0;
  for (int w = 0; w < 256 / kWave; ++w) total += s_wave[w];
  if (t < 256) {
    for (int w = 0; w < wave; ++w) incl += s_wave[w];
    if (mine > 0 && incl >= rank && incl - mine < rank) {  // exactly one thread
      int64_t run = incl - mine;
      for (int k = 0; k < per; ++k) {
        const int h = h0 + k;
        const int32_t c = h < n_bins ? summed(h) : 0;
        if (run + c >= rank) {
          s_bin = h;
          s_before = run;
          s_cnt = c;
          break;
        }
        run += c;
      }
    }
  }
  __syncthreads();
  if (t != 0) return;
  const int bin = s_bin;
  int bits = total != N ? QB_ERR_ROW_TOTALS : 0;
  if (bin < 0) bits |= QB_ERR_RANK;
  if (bits && err) atomicOr(err, bits);
  if (bin < 0 || bits) {
    q_out[int64_t(layer) * E + j] = __builtin_nanf("");
    return;
  }
  const double lo = double(bounds[2 * layer]);
  const double w = (double(bounds[2 * layer + 1]) - lo) / double(n_bins);
  const double frac = double(rank - s_before) / double(s_cnt);
  q_out[int64_t(layer) * E + j] = float(lo + w * (double(bin) + frac));
}

int launch_select_uniform_ws(int L, int64_t N, int E, int K, int n_bins, int64_t G, const uint8_t* ws,
                             int32_t* hist_u, float* q_out, float* b, float* bounds, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(k_select_uniform_ws, dim3(unsigned(E), unsigned(L)), dim3(kUWsThreads), 0, st, N, E, K, n_bins,
                     int(G), ws, uh_ws_layout(L, E, G, n_bins), hist_u, q_out, bounds, err);
  if (int rc = int(hipGetLastError())) return rc;
  hipLaunchKernelGGL(k_finalize, dim3(unsigned(L)), dim3(kFinThreads), 0, st, E, q_out, b, bounds, err);
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
