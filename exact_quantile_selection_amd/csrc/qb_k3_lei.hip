// qb_k3_lei.hip -- the K3 uniform-bin histogram pass and the LEI gradient
// offset.
//
// K3: "[Dev] Add global-batch quantile balancing" (Megatron-LM PR #6637),
// sections "Quantile estimator" and "Implementation": 1000 uniform bins per
// expert over [min(b) - 1, max(b) + 1], accumulated into an int32 [E, bins]
// histogram.  The fp32 margin is binned directly (no bf16 rounding).
// LEI: "Exact Quantile Balancing and Load-Error Injection for
// Mixture-of-Experts" (summary page), LEI paragraph: every token's gradient
// with respect to expert e's score is shifted by eta * rho_e, rho_e being
// that expert's relative load error over the batch.
//
// Layout of the K3 pass: E x n_bins counters do not fit in LDS, so each
// workgroup owns a slice of S experts (S = 64 for up to 1024 bins, 32 or 16
// for more bins or fewer experts) and a block of rows, and counts in packed
// 16-bit pairs (two experts per dword; <= 65535 rows per workgroup), about
// 128 KiB of LDS at 64 experts x 1000 bins.  S/4 lanes read the slice's
// S * 4 contiguous bytes of a row (256 B at S = 64), 64/(S/4) rows per load
// instruction; the row stride of the counter table is one more than a
// multiple of 64 dwords, so the lanes of different experts that hit the
// same bin land in different banks.  The counts are flushed once per
// workgroup into the int32 [E][n_bins] histogram with agent-scope atomics,
// or stored as the workgroup's partial rows in a workspace that the
// workspace select (qb_select.hip) sums.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "qb_device.hpp"
#include "qb_internal.hpp"

namespace qbk {

constexpr int kUHWaves = 16;
constexpr int kUHThreads = kUHWaves * kWave;
#ifndef QB_UH_REVERSE
#define QB_UH_REVERSE 1
#endif
#ifndef QB_UH_UNROLL
#define QB_UH_UNROLL 8
#endif
constexpr int kUHUnroll = QB_UH_UNROLL;  // rows per lane per trip
// workgroups per CU when the counter table takes at most 40 KiB
#ifndef QB_UH_SMALL_PER_CU
#define QB_UH_SMALL_PER_CU 4
#endif

template <int S>
struct UHShape {
  static constexpr int QPS = S / 4;                // lanes per row (one float4 each)
  static constexpr int RPI = kWave / QPS;          // rows per load instruction
  static constexpr int RPW = RPI * kUHUnroll;      // rows per wave trip
  static constexpr int STEP = kUHWaves * RPW;      // rows per workgroup trip
};

// Row stride (dwords) of the packed counter table for n_bins bins.
inline int uh_stride(int n_bins) { return (n_bins + 63) / 64 * 64 + 1; }

// hist_u == nullptr: instead of the atomic flush, the workgroup stores each
// expert's counts as its own partial row in the workspace ws (UhWs in
// qb_internal.hpp) for a select that sums them.
template <int S, bool ST = false>
__global__ __launch_bounds__(kUHThreads) void k_uniform_hist(
    const float* __restrict__ s, const float* __restrict__ alpha, int64_t N, int E,
    const float* __restrict__ bounds, int n_bins, int stride, int wg_per_slice, int32_t* __restrict__ hist_u,
    uint8_t* __restrict__ ws, UhWs wl) {
  using U = UHShape<S>;
  extern __shared__ uint32_t lds_u[];  // [S / 2][stride] packed pairs
  const int n_slices = E / S;
  const int per_layer = n_slices * wg_per_slice;
  const int layer = blockIdx.x / per_layer;
  const int rem = blockIdx.x - layer * per_layer;
  const int slice = rem % n_slices;
  const int g = rem / n_slices;
  s += int64_t(layer) * N * E + slice * S;
  alpha += int64_t(layer) * N;
  const int tid = threadIdx.x;
  const int words = (S / 2) * stride;
  for (int d = tid; d < words; d += kUHThreads) lds_u[d] = 0u;
  const float lo = bounds[2 * layer];
  const float hi = bounds[2 * layer + 1];
  const float width = hi - lo;
  const float inv_w = float(n_bins) / width;
  const float fbins = float(n_bins);
  __syncthreads();

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int q = lane % U::QPS;
  const int rsub = lane / U::QPS;
  uint32_t* rowp = lds_u + 2 * q * stride;  // experts 4q, 4q+1; 4q+2, 4q+3 one stride on
  auto load_rows = [&](int64_t base, float4 (&x)[kUHUnroll], float (&a)[kUHUnroll]) {
#pragma unroll
    for (int u = 0; u < kUHUnroll; ++u) {
      int64_t row = base + u * U::RPI + rsub;
      row = row < N ? row : N - 1;
      x[u] = (ST ? ld4_nt : ld4)(s + row * E + 4 * q);
      a[u] = alpha[row];
    }
  };
  // Block-cyclic trips of STEP rows: this workgroup takes g, g + G, ...
  // Every wave runs the workgroup's trip count (rows past N are clamped for
  // the loads and not counted).  Once per trip the waves meet at a bare
  // barrier; the upper half issues its loads before it and the lower half
  // after it, so one half's rows are in flight while the other half bins:
  // 217 us against 227 us with free-running waves at 1M x 256 and 1000
  // bins (34 against 36 us at 65,536 rows).  Two register sets per wave
  // (the next trip's rows loaded before this trip is binned) gained nothing
  // at 1M rows and cost 10 us at 65,536.  The barrier orders nothing: the
  // counters need no ordering until the flush, which a full barrier precedes.
  const int64_t trips = (N + U::STEP - 1) / U::STEP;
  const int64_t nT = trips > g ? (trips - 1 - g) / wg_per_slice + 1 : 0;
  const bool early = wave >= kUHWaves / 2;
  for (int64_t k = 0; k < nT; ++k) {
    // QB_UH_REVERSE: trips from the last to the first, so the rows pass 1
    // read last (still in the memory-side cache) are binned first
    const int64_t kt = QB_UH_REVERSE ? nT - 1 - k : k;
    const int64_t base = (int64_t(g) + kt * wg_per_slice) * U::STEP + int64_t(wave) * U::RPW;
    float4 x[kUHUnroll];
    float a[kUHUnroll];
    if (early) {
      load_rows(base, x, a);
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_barrier();
      load_rows(base, x, a);
    }
#pragma unroll
    for (int u = 0; u < kUHUnroll; ++u) {
      if (base + u * U::RPI + rsub < N) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float r = a[u] - comp(x[u], c);
          const float t = (r - lo) * inv_w;
          const int idx = !(t >= 0.0f) ? 0 : (t >= fbins ? n_bins - 1 : int(t));
          atomicAdd(rowp + (c >> 1) * stride + idx, (c & 1) ? 0x10000u : 1u);
        }
      }
    }
  }
  __syncthreads();
  if (hist_u == nullptr) {
    // Partial rows, one wave per dword row of the table (experts 2p and
    // 2p + 1 of the slice): a ballot over the row decides bytes or uint16
    // for each expert, then each lane stores 4 bins of each expert per step
    // (non-temporal: read once, by the select).
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    for (int p = wave; p < S / 2; p += kUHWaves) {
      const uint32_t* row = lds_u + p * stride;
      bool big0 = false, big1 = false;
      for (int b = lane; b < n_bins; b += kWave) {
        const uint32_t v = row[b];
        big0 |= (v & 0xFFFFu) > 255u;
        big1 |= (v >> 16) > 255u;
      }
      const bool w0 = __ballot(big0) != 0, w1 = __ballot(big1) != 0;
      const int64_t r0 = (int64_t(layer) * E + slice * S + 2 * p) * wg_per_slice + g;
      const int64_t r1 = r0 + wg_per_slice;  // expert 2p + 1
      if (lane == 0) {
        ws[wl.flag + r0] = w0 ? 1 : 0;
        ws[wl.flag + r1] = w1 ? 1 : 0;
      }
      for (int b = 4 * lane; b < n_bins; b += 4 * kWave) {
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = b + k < n_bins ? row[b + k] : 0u;
        const bool ws0[2] = {w0, w1};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t r = h ? r1 : r0;
          uint32_t c[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) c[k] = h ? (v[k] >> 16) : (v[k] & 0xFFFFu);
          if (ws0[h]) {
            uint2* dst = reinterpret_cast<uint2*>(ws + wl.p16 + r * wl.b16 + 2 * b);
            __builtin_nontemporal_store(c[0] | (c[1] << 16), &dst->x);
            __builtin_nontemporal_store(c[2] | (c[3] << 16), &dst->y);
          } else {
            uint32_t* dst = reinterpret_cast<uint32_t*>(ws + wl.p8 + r * wl.b8 + b);
            __builtin_nontemporal_store(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), dst);
          }
        }
      }
    }
    return;
  }
  // Flush: the G workgroups of a slice add into the same counters, so each
  // starts its walk at a different block of the table (by its index g).
  // A thread takes two adjacent bins of one dword row (two experts), and
  // for each expert adds both with one 64-bit atomic when the pair is
  // 8-byte aligned in the output (counts stay below 2^31, so the low half
  // never carries into the high one): the counts of a slice cover runs of
  // adjacent bins, so the atomics are about half as many.  The flush is a
  // tail of ~20 us at 1M x 256 either way (213-215 us with one atomic per
  // counter, 211-212 us with pairs).
  int32_t* out = hist_u + (int64_t(layer) * E + slice * S) * n_bins;
  const int halves = (n_bins + 1) / 2;  // bin pairs per row
  const int items = (S / 2) * halves;
  const int nblk = (items + kUHThreads - 1) / kUHThreads;
  const int b0 = g % nblk;
  auto add2 = [](int32_t* o, uint32_t a, uint32_t c, bool two) {
    if (two && (reinterpret_cast<uintptr_t>(o) & 7u) == 0) {
      if (a | c)
        atomicAdd(reinterpret_cast<unsigned long long*>(o), (unsigned long long)a | ((unsigned long long)c << 32));
    } else {
      if (a) atomicAdd(o, int(a));
      if (c) atomicAdd(o + 1, int(c));
    }
  };
  for (int k = 0; k < nblk; ++k) {
    int blk = b0 + k;
    blk = blk >= nblk ? blk - nblk : blk;
    const int e = blk * kUHThreads + tid;
    if (e >= items) continue;
    const int pair = e / halves;
    const int bin = 2 * (e - pair * halves);
    const bool two = bin + 1 < n_bins;
    const uint32_t v0 = lds_u[pair * stride + bin];
    const uint32_t v1 = two ? lds_u[pair * stride + bin + 1] : 0u;
    if ((v0 | v1) == 0u) continue;
    int32_t* o = out + int64_t(2 * pair) * n_bins + bin;
    add2(o, v0 & 0xFFFFu, v1 & 0xFFFFu, two);
    add2(o + n_bins, v0 >> 16, v1 >> 16, two);
  }
}

template <int S>
static int64_t uh_groups(int L, int64_t N, int E, int per_cu) {
  using U = UHShape<S>;
  const int n_slices = E / S;
  const int64_t trips = (N + U::STEP - 1) / U::STEP;
  const int64_t max_trips = std::max<int64_t>(1, 65535 / U::STEP);  // 16-bit counters
  int64_t G = (int64_t(device_cu_count()) * per_cu + int64_t(L) * n_slices - 1) / (int64_t(L) * n_slices);
  G = std::max(G, (trips + max_trips - 1) / max_trips);
  return std::max<int64_t>(1, std::min(G, trips));
}

// Largest bin count a slice width serves (launch_uniform_hist picks 64-expert
// slices only up to 1024 bins; the API allows 2048).
template <int S>
constexpr int uh_max_bins() { return S == 64 ? 1024 : 2048; }

// Allows k_uniform_hist<S> the dynamic LDS of the largest table any bin count
// it serves can need (at most 131,200 B), once per device and thread-safe, so
// a later call with more bins never launches past the allowed size.
template <int S, bool ST>
static int uh_allow_lds() {
  static std::atomic<uint64_t> done{0};  // bit d: set on device d
  static std::mutex mu;
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return int(ge);
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return int(hipSuccess);
  const size_t lds = size_t(S / 2) * size_t(uh_stride(uh_max_bins<S>())) * sizeof(uint32_t);
  std::lock_guard<std::mutex> lock(mu);
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return int(hipSuccess);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_uniform_hist<S, ST>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return int(e);
  }
  done.fetch_or(bit, std::memory_order_release);
  return int(hipSuccess);
}

// workgroups per CU that the table of S experts leaves room for (up to 4)
template <int S>
static int uh_per_cu(int n_bins) {
  const size_t lds = size_t(S / 2) * size_t(uh_stride(n_bins)) * sizeof(uint32_t);
  return lds > 80 * 1024 ? 1 : (lds > 40 * 1024 ? 2 : QB_UH_SMALL_PER_CU);
}

template <int S>
static int launch_uh(const float* s, const float* alpha, int L, int64_t N, int E, const float* bounds,
                     int n_bins, int32_t* hist_u, uint8_t* ws, hipStream_t st) {
  const int stride = uh_stride(n_bins);
  const size_t lds = size_t(S / 2) * size_t(stride) * sizeof(uint32_t);
  const int n_slices = E / S;
  const int64_t G = uh_groups<S>(L, N, E, uh_per_cu<S>(n_bins));
  const int64_t blocks = int64_t(L) * n_slices * G;
  // layers far larger than the Infinity Cache are read with non-temporal
  // loads (stream_pass) when the row segments are whole lines (S >= 32)
  if constexpr (S >= 32) {
    if (stream_pass(L, N, E)) {
      const int ea = uh_allow_lds<S, true>();
      if (ea != int(hipSuccess)) return ea;
      hipLaunchKernelGGL((k_uniform_hist<S, true>), dim3(unsigned(blocks)), dim3(kUHThreads), lds, st, s, alpha, N,
                         E, bounds, n_bins, stride, int(G), hist_u, ws, uh_ws_layout(L, E, G, n_bins));
      return int(hipGetLastError());
    }
  }
  const int ea = uh_allow_lds<S, false>();
  if (ea != int(hipSuccess)) return ea;
  hipLaunchKernelGGL((k_uniform_hist<S>), dim3(unsigned(blocks)), dim3(kUHThreads), lds, st, s, alpha, N, E,
                     bounds, n_bins, stride, int(G), hist_u, ws, uh_ws_layout(L, E, G, n_bins));
  return int(hipGetLastError());
}

// Wider slices read longer row segments (whole lines from 32 experts) but
// give each workgroup a larger table to clear and merge; they are used when
// every workgroup still gets enough rows: 64-expert slices from 1024 rows
// per workgroup when the tables leave through the workspace, from 2048 when
// they are flushed with global atomics (a larger tail per workgroup), and
// 32-expert slices (more than 1024 bins) from 8192.  Measured on one MI355X
// with 1000 bins and 256 experts: at 65,536 tokens (1024 rows per
// workgroup) the workspace binning pass takes 20.8-21.1 us with 64-expert
// slices, 22.4-23.3 with 32 and 27.5-28.3 with 16 (K3 step 48.9-49.3
// against 53.2-54.3 us), while the atomic one took 47 us with 64-expert
// slices against 35 with 16; at 131,072 tokens 52 us with 64-expert slices
// against 59-63 us with 16 (atomic merge).
#ifndef QB_UH_MIN_ROWS
#define QB_UH_MIN_ROWS 8192
#endif
#ifndef QB_UH_MIN_ROWS64_WS
#define QB_UH_MIN_ROWS64_WS 1024
#endif
#ifndef QB_UH_MIN_ROWS64
#define QB_UH_MIN_ROWS64 2048
#endif

// Slice width of the binning pass for a shape; ws: the tables leave
// through the workspace (else by global atomics).
static int uh_slice(int L, int64_t N, int E, int n_bins, bool ws) {
  const int64_t min64 = ws ? QB_UH_MIN_ROWS64_WS : QB_UH_MIN_ROWS64;
  if (E >= 64 && n_bins <= 1024 && N / uh_groups<64>(L, N, E, 1) >= min64) return 64;
  if (E >= 32 && N / uh_groups<32>(L, N, E, 1) >= QB_UH_MIN_ROWS) return 32;
  return 16;
}

int64_t uniform_hist_groups(int L, int64_t N, int E, int n_bins) {
  switch (uh_slice(L, N, E, n_bins, true)) {
    case 64: return uh_groups<64>(L, N, E, uh_per_cu<64>(n_bins));
    case 32: return uh_groups<32>(L, N, E, uh_per_cu<32>(n_bins));
  }
  return uh_groups<16>(L, N, E, uh_per_cu<16>(n_bins));
}

static int launch_uniform_hist_any(const float* s, const float* alpha, int L, int64_t N, int E,
                                   const float* bounds, int n_bins, int32_t* hist_u, uint8_t* ws, hipStream_t st) {
  switch (uh_slice(L, N, E, n_bins, ws != nullptr)) {
    case 64: return launch_uh<64>(s, alpha, L, N, E, bounds, n_bins, hist_u, ws, st);
    case 32: return launch_uh<32>(s, alpha, L, N, E, bounds, n_bins, hist_u, ws, st);
  }
  return launch_uh<16>(s, alpha, L, N, E, bounds, n_bins, hist_u, ws, st);
}

int launch_uniform_hist(const float* s, const float* alpha, int L, int64_t N, int E,
                        const float* bounds, int n_bins, int32_t* hist_u, hipStream_t st) {
  return launch_uniform_hist_any(s, alpha, L, N, E, bounds, n_bins, hist_u, nullptr, st);
}

int launch_uniform_hist_ws(const float* s, const float* alpha, int L, int64_t N, int E, const float* bounds,
                           int n_bins, uint8_t* ws, hipStream_t st) {
  return launch_uniform_hist_any(s, alpha, L, N, E, bounds, n_bins, nullptr, ws, st);
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
// Mixture-of-Experts", summary page, LEI paragraph: each token of a local
// batch gets eta * rho_e added to its gradient for expert e's score; the
// page's "normalized" variant limits the size of the residual vector with
// tanh while leaving its direction and its zero sum unchanged).  Microbatch
// c = rows [c n_mb, (c+1) n_mb):
//   rho_e  = fl32(((double)load[c][e] - M) / M),  M = n_mb K / E
//   bounded: rho_e = fl32((double)rho_e * tanh(|rho|) / |rho|), |rho| the
//            L2 norm over experts in float64 (sum in expert order)
//   add_e  = fl32(eta * rho_e)
//   g'     = fl32(g + add_e);  dlogit = fl32(g' * fl32(s * fl32(1 - s)))
// grid (G, C): blockIdx.y is the microbatch.
// Float4 groups per thread and trip, and workgroups per CU of the grid (up
// to the work available): many small workgroups keep enough reads in flight
// (at 262,144 x 256: 189 us with 64 per CU against 236 us with 8).
#ifndef QB_LEI_U
#define QB_LEI_U 4
#endif
// g' and the logit gradient are streamed out and not read again here:
// non-temporal stores (unbounded 177 -> 173 us, bounded 190 -> 182 us at
// 262,144 x 256, one MI355X)
typedef float lei_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ lei_f4 f4v(const float4& a) {
  lei_f4 r;
  r.x = a.x;
  r.y = a.y;
  r.z = a.z;
  r.w = a.w;
  return r;
}
#ifndef QB_LEI_WG_PER_CU
#define QB_LEI_WG_PER_CU 64
#endif

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
  // Unbounded, each thread computes the offsets of its own four experts
  // (below); the bounded rescale needs the norm over all E, so its table
  // goes through LDS.  (bounded is uniform over the grid.)
  if (bounded) {
    for (int e = threadIdx.x; e < E; e += kLeiThreads) add[e] = float((double(load[e]) - M) / M);
    __syncthreads();
    if (threadIdx.x == 0) {
      double n2 = 0.0;
      for (int e = 0; e < E; ++e) n2 += double(add[e]) * double(add[e]);
      const double norm = sqrt(n2);
      s_lambda = norm > 0.0 ? tanh(norm) / norm : 1.0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kLeiThreads) add[e] = eta * float(double(add[e]) * s_lambda);
    __syncthreads();
  }
  // The float4 stride of the grid is a multiple of E/4, so every thread
  // keeps the same four experts.
  const int64_t n4 = n_mb * E / 4;
  const int64_t base4 = int64_t(c) * n4;
  const int64_t stride = int64_t(gridDim.x) * kLeiThreads;
  const int64_t i0 = int64_t(blockIdx.x) * kLeiThreads + threadIdx.x;
  const int e0 = int((i0 * 4) % E);
  float a0, a1, a2, a3;
  if (!bounded) {
    a0 = eta * float((double(load[e0]) - M) / M);
    a1 = eta * float((double(load[e0 + 1]) - M) / M);
    a2 = eta * float((double(load[e0 + 2]) - M) / M);
    a3 = eta * float((double(load[e0 + 3]) - M) / M);
  } else {
    a0 = add[e0];
    a1 = add[e0 + 1];
    a2 = add[e0 + 2];
    a3 = add[e0 + 3];
  }
  const float4* g4 = reinterpret_cast<const float4*>(g) + base4;
  const float4* s4 = s ? reinterpret_cast<const float4*>(s) + base4 : nullptr;
  float4* go4 = g_out ? reinterpret_cast<float4*>(g_out) + base4 : nullptr;
  float4* d4 = dlogits ? reinterpret_cast<float4*>(dlogits) + base4 : nullptr;
  // four strided elements per thread and trip: all loads issued before any
  // store, so each thread keeps 8 (or 4) 16-byte reads in flight
  constexpr int U = QB_LEI_U;
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
      if (go4) __builtin_nontemporal_store(f4v(v[u]), reinterpret_cast<lei_f4*>(go4 + k));
      if (d4) {
        float4 d;
        d.x = v[u].x * (p[u].x * (1.0f - p[u].x));
        d.y = v[u].y * (p[u].y * (1.0f - p[u].y));
        d.z = v[u].z * (p[u].z * (1.0f - p[u].z));
        d.w = v[u].w * (p[u].w * (1.0f - p[u].w));
        __builtin_nontemporal_store(f4v(d), reinterpret_cast<lei_f4*>(d4 + k));
      }
    }
  }
}

int launch_lei_bwd(const float* g, const float* s, const int32_t* load_mb, int64_t N, int E, int K,
                   int64_t n_mb, float eta, int bounded, float* g_out, float* dlogits, hipStream_t st) {
  const int64_t C = N / n_mb;
  const int64_t n4 = n_mb * E / 4;
  const int64_t want = std::max<int64_t>(1, (n4 + kLeiThreads - 1) / kLeiThreads);
  const int64_t cap = std::max<int64_t>(1, int64_t(device_cu_count()) * QB_LEI_WG_PER_CU / C);
  const unsigned gx = unsigned(std::min(want, cap));
  hipLaunchKernelGGL(k_lei_bwd, dim3(gx, unsigned(C)), dim3(kLeiThreads), 0, st, g, s, load_mb, n_mb, E, K, eta,
                     bounded, g_out, dlogits);
  return int(hipGetLastError());
}

}  // namespace qbk
