// qb_shard.hip -- one-GPU emulation of the data-parallel update: R emulated
// ranks, each holding its own copy of every per-rank buffer (rank r's copy at
// offset r * M), and the two ways the pages compare to combine them.
//
// "Exact Quantile Balancing and Load-Error Injection for Mixture-of-Experts"
// (summary page), background paragraph: no data-parallel rank sees the whole
// margin distribution; the MARIN implementation averages rank-local
// quantiles, which do not commute with averaging, so its result depends on
// the sharding; a histogram summed over ranks is partition-invariant.  EQB
// paragraph: two all-reduces of 256-bin histograms per update.
//
//  * k_allreduce_sum: every rank's copy becomes the elementwise sum of all
//    copies (an all-reduce with integer addition, so any summation order
//    gives the same bytes).
//  * k_rank_average: the rank-averaged update, q_j = fl32(sum_r (double)
//    q_j^(r) / R) in rank order, then b_j = fl32((double)q_j - mean_j
//    (double)q_j) with the mean a float64 sum in expert order / E, and
//    bounds = [fl32(min b - 1), fl32(max b + 1)] (the same centring and
//    bounds as the EQB update).
#include "qb_device.hpp"
#include "qb_internal.hpp"

namespace qbk {

constexpr int kArThreads = 256;

__global__ __launch_bounds__(kArThreads) void k_allreduce_sum(int32_t* __restrict__ buf, int R, int64_t M) {
  const int64_t stride = int64_t(gridDim.x) * kArThreads;
  for (int64_t m = int64_t(blockIdx.x) * kArThreads + threadIdx.x; m < M; m += stride) {
    int32_t sum = 0;
    for (int r = 0; r < R; ++r) sum += buf[int64_t(r) * M + m];
    for (int r = 0; r < R; ++r) buf[int64_t(r) * M + m] = sum;
  }
}

// One workgroup: thread j averages expert j's rank-local quantiles; thread 0
// then forms the float64 mean in expert order and the bounds.
__global__ __launch_bounds__(kArThreads) void k_rank_average(const float* __restrict__ q, int R, int E,
                                                             float* __restrict__ b, float* __restrict__ bounds) {
  extern __shared__ float s_q[];  // E floats
  for (int j = threadIdx.x; j < E; j += kArThreads) {
    double sum = 0.0;
    for (int r = 0; r < R; ++r) sum += double(q[int64_t(r) * E + j]);
    s_q[j] = float(sum / double(R));
  }
  __syncthreads();
  __shared__ double s_mean;
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int j = 0; j < E; ++j) sum += double(s_q[j]);
    s_mean = sum / double(E);
  }
  __syncthreads();
  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int j = threadIdx.x; j < E; j += kArThreads) {
    const float bj = float(double(s_q[j]) - s_mean);
    b[j] = bj;
    lo = fminf(lo, bj);
    hi = fmaxf(hi, bj);
  }
  __shared__ float s_lo[kArThreads], s_hi[kArThreads];
  s_lo[threadIdx.x] = lo;
  s_hi[threadIdx.x] = hi;
  __syncthreads();
  if (threadIdx.x == 0 && bounds) {
    for (int t = 1; t < kArThreads; ++t) {
      lo = fminf(lo, s_lo[t]);
      hi = fmaxf(hi, s_hi[t]);
    }
    bounds[0] = lo - 1.0f;
    bounds[1] = hi + 1.0f;
  }
}

int launch_allreduce_sum(int32_t* buf, int R, int64_t M, hipStream_t st) {
  const int64_t want = (M + kArThreads - 1) / kArThreads;
  const int64_t cap = int64_t(device_cu_count()) * 8;
  const unsigned blocks = unsigned(want < cap ? want : cap);
  hipLaunchKernelGGL(k_allreduce_sum, dim3(blocks), dim3(kArThreads), 0, st, buf, R, M);
  return int(hipGetLastError());
}

int launch_rank_average(const float* q, int R, int E, float* b, float* bounds, hipStream_t st) {
  hipLaunchKernelGGL(k_rank_average, dim3(1u), dim3(kArThreads), size_t(E) * sizeof(float), st, q, R, E, b,
                     bounds);
  return int(hipGetLastError());
}

}  // namespace qbk
