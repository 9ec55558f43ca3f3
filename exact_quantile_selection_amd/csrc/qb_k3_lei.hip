// qb_k3_lei.hip -- the K3 uniform-bin histogram pass and the LEI gradient
// offset.
//
// K3: "[Dev] Add global-batch quantile balancing" (Megatron-LM PR #6637),
// sections "Quantile estimator" and "Implementation": 1000 uniform bins per
// expert over [min(b) - 1, max(b) + 1], accumulated into an int32 [E, bins]
// histogram.  The fp32 margin is binned directly (no bf16 rounding).
// LEI: "Exact Quantile Balancing and Load-Error Injection for
// Mixture-of-Experts" (summary page), LEI paragraph: add eta * rho_e to the
// score gradient of expert e for every token of the batch.
//
// Layout of the K3 pass: E x 1000 int32 counters do not fit in LDS, so each
// workgroup owns a slice of 16 experts (16 * n_bins int32 in LDS, 64 KB at
// 1000 bins, two workgroups per CU) and a chunk of rows; 4 lanes read the
// slice's 64 contiguous bytes of a row, 16 rows per load instruction.
#include <algorithm>

#include "qb_device.hpp"
#include "qb_internal.hpp"

namespace qbk {

constexpr int kUHThreads = 512;
constexpr int kUHWaves = kUHThreads / kWave;
constexpr int kUHSlice = 16;                 // experts per workgroup
constexpr int kUHRPI = kWave / (kUHSlice / 4);  // rows per load instruction
constexpr int kUHUnroll = 4;
constexpr int kUHStep = kUHWaves * kUHRPI * kUHUnroll;

__global__ __launch_bounds__(kUHThreads) void k_uniform_hist(
    const float* __restrict__ s, const float* __restrict__ alpha, int64_t N, int E,
    const float* __restrict__ bounds, int n_bins, int wg_per_layer, int32_t* __restrict__ hist_u) {
  extern __shared__ int32_t lds_u[];  // [kUHSlice][n_bins]
  const int n_slices = E / kUHSlice;
  const int per_layer = n_slices * wg_per_layer;
  const int layer = blockIdx.x / per_layer;
  const int rem = blockIdx.x - layer * per_layer;
  const int slice = rem % n_slices;
  const int g = rem / n_slices;
  s += int64_t(layer) * N * E + slice * kUHSlice;
  alpha += int64_t(layer) * N;
  const int tid = threadIdx.x;
  for (int d = tid; d < kUHSlice * n_bins; d += kUHThreads) lds_u[d] = 0;
  const float lo = bounds[2 * layer];
  const float hi = bounds[2 * layer + 1];
  const float width = hi - lo;
  const float inv_w = float(n_bins) / width;
  const float fbins = float(n_bins);
  __syncthreads();

  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int q4 = lane & 3;
  const int rsub = lane >> 2;
  int32_t* cnt = lds_u + 4 * q4 * n_bins;
  // Block-cyclic trips of kUHStep rows: this workgroup takes g, g + G, ...
  for (int64_t base = int64_t(g) * kUHStep + int64_t(wave) * kUHRPI * kUHUnroll; base < N;
       base += int64_t(wg_per_layer) * kUHStep) {
    float4 x[kUHUnroll];
    float a[kUHUnroll];
#pragma unroll
    for (int u = 0; u < kUHUnroll; ++u) {
      int64_t row = base + u * kUHRPI + rsub;
      row = row < N ? row : N - 1;
      x[u] = ld4(s + row * E + 4 * q4);
      a[u] = alpha[row];
    }
#pragma unroll
    for (int u = 0; u < kUHUnroll; ++u) {
      if (base + u * kUHRPI + rsub < N) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float r = a[u] - comp(x[u], c);
          const float t = (r - lo) * inv_w;
          const int idx = !(t >= 0.0f) ? 0 : (t >= fbins ? n_bins - 1 : int(t));
          atomicAdd(cnt + c * n_bins + idx, 1);
        }
      }
    }
  }
  __syncthreads();
  int32_t* out = hist_u + (int64_t(layer) * E + slice * kUHSlice) * n_bins;
  for (int d = tid; d < kUHSlice * n_bins; d += kUHThreads)
    if (lds_u[d]) atomicAdd(out + d, lds_u[d]);
}

int launch_uniform_hist(const float* s, const float* alpha, int L, int64_t N, int E,
                        const float* bounds, int n_bins, int32_t* hist_u, hipStream_t st) {
  // Row-trip workgroups per (layer, slice) so that all layers' slices make
  // about two workgroups per CU.
  const int n_slices = E / kUHSlice;
  const int64_t trips = (N + kUHStep - 1) / kUHStep;
  const int64_t per = std::max<int64_t>(
      1, (2 * int64_t(device_cu_count()) + int64_t(L) * n_slices - 1) / (int64_t(L) * n_slices));
  const int G = int(std::min<int64_t>(per, trips));
  const int64_t blocks = int64_t(L) * n_slices * G;
  const size_t lds = size_t(kUHSlice) * size_t(n_bins) * sizeof(int32_t);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_uniform_hist),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return int(e);
  }
  hipLaunchKernelGGL(k_uniform_hist, dim3(unsigned(blocks)), dim3(kUHThreads), lds, st, s, alpha, N,
                     E, bounds, n_bins, G, hist_u);
  return int(hipGetLastError());
}

// ---------------------------------------------------------------------------
constexpr int kLeiThreads = 256;

__global__ __launch_bounds__(kLeiThreads) void k_lei(float* __restrict__ g,
                                                     const int32_t* __restrict__ load, int64_t N,
                                                     int E, int K, float eta) {
  __shared__ float add[256];
  const double M = double(N) * double(K) / double(E);
  for (int e = threadIdx.x; e < E; e += kLeiThreads) {
    const float rho = float((double(load[e]) - M) / M);
    add[e] = eta * rho;
  }
  __syncthreads();
  // The float4 stride of the grid is a multiple of E/4, so every thread
  // keeps the same four experts.
  const int64_t n4 = N * E / 4;
  const int64_t stride = int64_t(gridDim.x) * kLeiThreads;
  const int64_t i0 = int64_t(blockIdx.x) * kLeiThreads + threadIdx.x;
  const int e0 = int((i0 * 4) % E);
  const float a0 = add[e0], a1 = add[e0 + 1], a2 = add[e0 + 2], a3 = add[e0 + 3];
  float4* g4 = reinterpret_cast<float4*>(g);
  for (int64_t i = i0; i < n4; i += stride) {
    float4 v = g4[i];
    v.x = v.x + a0;
    v.y = v.y + a1;
    v.z = v.z + a2;
    v.w = v.w + a3;
    g4[i] = v;
  }
}

int launch_lei(float* g, const int32_t* load, int64_t N, int E, int K, float eta, hipStream_t st) {
  const int64_t n4 = N * E / 4;
  const int64_t blocks = std::min<int64_t>(int64_t(device_cu_count()) * 8,
                                           std::max<int64_t>(1, (n4 + kLeiThreads - 1) / kLeiThreads));
  hipLaunchKernelGGL(k_lei, dim3(unsigned(blocks)), dim3(kLeiThreads), 0, st, g, load, N, E, K, eta);
  return int(hipGetLastError());
}

// LEI per microbatch, optionally bounded, and the gradient through the
// sigmoid ("Exact Quantile Balancing and Load-Error Injection for
// Mixture-of-Experts", summary page, LEI paragraph: add eta * rho_e to the
// score gradient of expert e for every token of the local batch; the
// shipped variant bounds the residual with a tanh rescale that keeps its
// direction and zero-centring).  Microbatch c = rows [c n_mb, (c+1) n_mb):
//   rho_e  = fl32(((double)load[c][e] - M) / M),  M = n_mb K / E
//   bounded: rho_e = fl32((double)rho_e * tanh(|rho|) / |rho|), |rho| the
//            L2 norm over experts in float64 (sum in expert order)
//   add_e  = fl32(eta * rho_e)
//   g'     = fl32(g + add_e);  dlogit = fl32(g' * fl32(s * fl32(1 - s)))
// grid (G, C): blockIdx.y is the microbatch.
__global__ __launch_bounds__(kLeiThreads) void k_lei_bwd(const float* __restrict__ g,
                                                         const float* __restrict__ s,
                                                         const int32_t* __restrict__ load_mb, int64_t n_mb,
                                                         int E, int K, float eta, int bounded,
                                                         float* g_out, float* __restrict__ dlogits) {
  __shared__ float add[256];
  __shared__ double s_lambda;
  const int c = blockIdx.y;
  const int32_t* load = load_mb + int64_t(c) * E;
  const double M = double(n_mb) * double(K) / double(E);
  for (int e = threadIdx.x; e < E; e += kLeiThreads) add[e] = float((double(load[e]) - M) / M);
  __syncthreads();
  if (bounded) {
    if (threadIdx.x == 0) {
      double n2 = 0.0;
      for (int e = 0; e < E; ++e) n2 += double(add[e]) * double(add[e]);
      const double norm = sqrt(n2);
      s_lambda = norm > 0.0 ? tanh(norm) / norm : 1.0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kLeiThreads) add[e] = float(double(add[e]) * s_lambda);
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += kLeiThreads) add[e] = eta * add[e];
  __syncthreads();
  // The float4 stride of the grid is a multiple of E/4, so every thread
  // keeps the same four experts.
  const int64_t n4 = n_mb * E / 4;
  const int64_t base4 = int64_t(c) * n4;
  const int64_t stride = int64_t(gridDim.x) * kLeiThreads;
  const int64_t i0 = int64_t(blockIdx.x) * kLeiThreads + threadIdx.x;
  const int e0 = int((i0 * 4) % E);
  const float a0 = add[e0], a1 = add[e0 + 1], a2 = add[e0 + 2], a3 = add[e0 + 3];
  const float4* g4 = reinterpret_cast<const float4*>(g) + base4;
  const float4* s4 = s ? reinterpret_cast<const float4*>(s) + base4 : nullptr;
  float4* go4 = g_out ? reinterpret_cast<float4*>(g_out) + base4 : nullptr;
  float4* d4 = dlogits ? reinterpret_cast<float4*>(dlogits) + base4 : nullptr;
  // four strided elements per thread and trip: all loads issued before any
  // store, so each thread keeps 8 (or 4) 16-byte reads in flight
  constexpr int U = 4;
  for (int64_t i = i0; i < n4; i += U * stride) {
    float4 v[U], p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = i + u * stride;
      if (k < n4) {
        v[u] = g4[k];
        if (d4) p[u] = s4[k];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = i + u * stride;
      if (k >= n4) continue;
      v[u].x = v[u].x + a0;
      v[u].y = v[u].y + a1;
      v[u].z = v[u].z + a2;
      v[u].w = v[u].w + a3;
      if (go4) go4[k] = v[u];
      if (d4) {
        float4 d;
        d.x = v[u].x * (p[u].x * (1.0f - p[u].x));
        d.y = v[u].y * (p[u].y * (1.0f - p[u].y));
        d.z = v[u].z * (p[u].z * (1.0f - p[u].z));
        d.w = v[u].w * (p[u].w * (1.0f - p[u].w));
        d4[k] = d;
      }
    }
  }
}

int launch_lei_bwd(const float* g, const float* s, const int32_t* load_mb, int64_t N, int E, int K,
                   int64_t n_mb, float eta, int bounded, float* g_out, float* dlogits, hipStream_t st) {
  const int64_t C = N / n_mb;
  const int64_t n4 = n_mb * E / 4;
  const int64_t want = std::max<int64_t>(1, (n4 + kLeiThreads - 1) / kLeiThreads);
  const int64_t cap = std::max<int64_t>(1, int64_t(device_cu_count()) * 8 / C);
  const unsigned gx = unsigned(std::min(want, cap));
  hipLaunchKernelGGL(k_lei_bwd, dim3(gx, unsigned(C)), dim3(kLeiThreads), 0, st, g, s, load_mb, n_mb, E, K, eta,
                     bounded, g_out, dlogits);
  return int(hipGetLastError());
}

}  // namespace qbk
