// qb_radix.hip -- streaming byte histograms of the bf16 margin keys from a
// precomputed alpha: the high-byte pass, and the low-byte pass restricted to
// each expert's selected high byte.
//
// Method: "Exact Quantile Balancing and Load-Error Injection for
// Mixture-of-Experts" (summary page), EQB paragraph: histogram the high byte
// into 256 bins, locate the bin holding the rank, then histogram the low byte
// within that bin; concatenating the bytes gives the exact quantile.
//
// Layout on gfx950: lane l of a wave owns float4 column block (quad)
// l % (E/4) of its row, so one load instruction covers 64*16 contiguous bytes
// (one row at E=256) and a wave trip reads RHShape::U load instructions
// (16 consecutive rows at E=256).  Trips are block-cyclic over the
// workgroups, so the workgroups in flight read neighbouring rows; half of a
// workgroup's waves load while the other half counts.
// Counters are the packed 16-bit LDS histogram of qb_device.hpp (bank swizzle
// by quad), flushed once per workgroup.  A lane's experts are fixed for the
// whole kernel, so the low-byte pass keeps their selected high bytes in
// registers and filters with one compare per element.
#include <algorithm>

#include "qb_device.hpp"
#include "qb_internal.hpp"

// Rows per workgroup at most (16-bit LDS counters hold 65535); smaller
// values give more, shorter-lived workgroups.
#ifndef QB_RH_MAXROWS
#define QB_RH_MAXROWS 65535
#endif

namespace qbk {

// vector types the non-temporal store builtin accepts
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#ifndef QB_RH_WAVES
#define QB_RH_WAVES 16
#endif
constexpr int kRHWaves = QB_RH_WAVES;
constexpr int kRHThreads = kRHWaves * kWave;

template <int E>
struct RHShape {
  static constexpr int QPR = E / 4;            // lanes per row
  static constexpr int RPI = kWave / QPR;      // rows per load instruction
  // rows per lane per trip: 16 at E = 256 (one row per load instruction);
  // 8 for narrower rows, whose row offsets take more registers per lane
  static constexpr int U = E >= 256 ? 16 : 8;
  static constexpr int RPW = RPI * U;          // rows per wave trip
  static constexpr int STEP = kRHWaves * RPW;  // rows per workgroup trip
  static_assert(QPR <= kWave && (kWave % QPR) == 0, "row split");
};

// WS: instead of adding its counts into the global histogram with atomics,
// the workgroup stores them, dense, as its own partial histogram row per
// expert in the workspace (LoWs in qb_internal.hpp: bytes when all 256
// counts of the row are <= 255, uint16 otherwise, and a flag saying which),
// for a select that sums the partials (no atomics, no zeroing).
template <int E, bool LO, bool WS>
__global__ __launch_bounds__(kRHThreads) void k_radix_hist(
    const float* __restrict__ s, const float* __restrict__ alpha, int64_t N, int wg_per_layer,
    const int32_t* __restrict__ sel_hi, int32_t* __restrict__ hist, uint8_t* __restrict__ ws,
    int64_t ws_flag, int64_t ws_p16) {
  using S = RHShape<E>;
  __shared__ uint32_t lds_hist[(E / 2) * 256];
  const int tid = threadIdx.x;
  const int layer = blockIdx.x / wg_per_layer;
  const int g = blockIdx.x - layer * wg_per_layer;
  s += int64_t(layer) * N * E;
  alpha += int64_t(layer) * N;

  hist16_zero<E>(lds_hist, tid, kRHThreads);

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int quad = lane % S::QPR;
  const int rsub = lane / S::QPR;
  const uint32_t swz = hist16_swizzle2(quad);               // high bytes of a key pair
  const uint32_t swzl = uint32_t(quad & 63) * 0x00010001u;  // low bytes of a key pair
  uint32_t* rowp = lds_hist + quad * 512;
  // Selected high byte of each of the lane's four experts; an invalid
  // selection (< 0) becomes 0x100, which no byte equals.
  uint32_t sel[4] = {0x100u, 0x100u, 0x100u, 0x100u};
  if constexpr (LO) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int v = sel_hi[int64_t(layer) * E + 4 * quad + c];
      sel[c] = (v >= 0 && v < 256) ? uint32_t(v) : 0x100u;
      // Materialise the value here: first used inside the row loop, the
      // load would otherwise be waited for there with a full vmcnt(0) on
      // every trip, draining the rows in flight.
      asm volatile("" : "+v"(sel[c]));
    }
  }
  __syncthreads();

  // Full trips (every row < N): addresses from the wave-uniform row base
  // with 32-bit lane offsets, no clamps and no per-row tests, so the loop
  // body is straight-line and each set's loads are waited for one by one.
  auto load_full = [&](int64_t base, float4 (&x)[S::U], float (&a)[S::U]) {
    const float* sw = s + base * E;
    const float* aw = alpha + base;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      x[u] = ld4(sw + uint32_t((u * S::RPI + rsub) * E + 4 * quad));
      a[u] = aw[u * S::RPI + rsub];
    }
  };
  auto count1 = [&](const float4& x, float a) {
    const uint32_t k01 = key2(bf16x2_rne(a - x.x, a - x.y));
    const uint32_t k23 = key2(bf16x2_rne(a - x.z, a - x.w));
    if constexpr (!LO) {
      hist16_add_hi(lds_hist, quad, 0, k01 ^ swz);
      hist16_add_hi(lds_hist, quad, 2, k23 ^ swz);
    } else {
      // low byte of the key, swizzled like the high-byte histogram
      const uint32_t l01 = k01 ^ swzl, l23 = k23 ^ swzl;
      if (((k01 >> 8) & 0xFFu) == sel[0]) atomicAdd(rowp + (l01 & 0xFFu), 1u);
      if ((k01 >> 24) == sel[1]) atomicAdd(rowp + ((l01 >> 16) & 0xFFu), 0x10000u);
      if (((k23 >> 8) & 0xFFu) == sel[2]) atomicAdd(rowp + 256 + (l23 & 0xFFu), 1u);
      if ((k23 >> 24) == sel[3]) atomicAdd(rowp + 256 + ((l23 >> 16) & 0xFFu), 0x10000u);
    }
  };
  // Block-cyclic trips: this workgroup takes trips g, g + G, g + 2G, ...
  // The loop runs over the trips whose rows are all below N, the same count
  // for every wave, and the waves meet at a bare barrier once per trip: kept
  // in step, the workgroup reads each block of rows together (190 us against
  // 197 us for 1M x 256 when the waves drift apart).  The upper half of the
  // waves issues its loads before the barrier and the lower half after it,
  // so one half's rows are in flight while the other half counts.  With 16
  // rows per lane in one register set this takes 186-187 us; two sets of 8
  // (the next trip loaded while this one is counted) took 190-191 us.  The
  // barrier orders nothing (the counters need no ordering until the flush,
  // which a full barrier precedes).  The workgroup's last trip, if partial,
  // runs after the loop.
  const int64_t full_trips = N / S::STEP;
  const int64_t nF = full_trips > g ? (full_trips - 1 - g) / wg_per_layer + 1 : 0;
  auto trip_base = [&](int64_t k) { return (int64_t(g) + k * wg_per_layer) * S::STEP + int64_t(wave) * S::RPW; };
  const bool early = wave >= kRHWaves / 2;
  float4 x[S::U];
  float a[S::U];
  for (int64_t k = 0; k < nF; ++k) {
    if (early) {
      load_full(trip_base(k), x, a);
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_barrier();
      load_full(trip_base(k), x, a);
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) count1(x[u], a[u]);
  }
  const int64_t base = trip_base(nF);
  if (base < N) {
    // the partial trip: rows clamped to N - 1 for the loads, not counted
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      int64_t row = base + u * S::RPI + rsub;
      row = row < N ? row : N - 1;
      x[u] = ld4(s + row * E + 4 * quad);
      a[u] = alpha[row];
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u)
      if (base + u * S::RPI + rsub < N) count1(x[u], a[u]);
  }
  __syncthreads();
  if constexpr (WS) {
    // Item i covers bins 8k .. 8k+7 (k = i & 31) of dword row pair = i >> 5
    // (experts 2 pair and 2 pair + 1).  Its eight counters are one aligned
    // 8-dword block of LDS, permuted by the row's bank swizzle
    // (quad = pair >> 1: c[m] holds bin 8k + (m ^ (quad & 7))).  The 32
    // items of a pair are one half of a wave, so a half-wave ballot tells
    // whether any of an expert's 256 counts exceeds 255: if none does, the
    // row leaves as 8 bytes per item, else as 8 uint16 (16 bytes) per item.
    // Lane k = 0 writes the row's flag.  A workgroup writes 64 KiB at
    // E = 256 when every row fits in bytes, half the uint16 partials.  The
    // rows leave with non-temporal stores (read once, by the select): at the
    // end of the pass less dirty data waits in L2 (182 -> 180 us at 1M).
    const int G = wg_per_layer;
    const int64_t row_base = int64_t(layer) * E * G + g;  // row of expert j: row_base + j * G
    uint8_t* flag = ws + ws_flag;
    uint16_t* p16 = reinterpret_cast<uint16_t*>(ws + ws_p16);
    for (int i = tid; i < (E / 2) * 32; i += kRHThreads) {
      const int pair = i >> 5, k = i & 31;
      const int sw = (pair >> 1) & 63;
      const uint4* src = reinterpret_cast<const uint4*>(lds_hist + pair * 256 + ((8 * k) ^ (sw & 0xF8)));
      const uint4 v0 = src[0], v1 = src[1];
      uint32_t c[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      // c[m] <- c[m ^ (sw & 7)], one XOR bit at a time
#pragma unroll
      for (int bit = 4; bit >= 1; bit >>= 1) {
        if (sw & bit) {
#pragma unroll
          for (int m = 0; m < 8; ++m)
            if ((m & bit) == 0) {
              const uint32_t t = c[m];
              c[m] = c[m | bit];
              c[m | bit] = t;
            }
        }
      }
      // expert 2 pair: the low halves of c; expert 2 pair + 1: the high halves
      uint32_t big_lo = 0, big_hi = 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        big_lo |= c[m] & 0xFF00u;
        big_hi |= c[m] & 0xFF000000u;
      }
      const uint64_t bal_lo = __ballot(big_lo != 0), bal_hi = __ballot(big_hi != 0);
      const int half = (tid & (kWave - 1)) >> 5;  // which pair of the wave
      const bool wide_lo = uint32_t(bal_lo >> (32 * half)) != 0;
      const bool wide_hi = uint32_t(bal_hi >> (32 * half)) != 0;
      const int64_t r_lo = row_base + int64_t(2 * pair) * G, r_hi = r_lo + G;
      if (wide_lo) {
        u32x4 o;
        o.x = (c[0] & 0xFFFFu) | (c[1] << 16);
        o.y = (c[2] & 0xFFFFu) | (c[3] << 16);
        o.z = (c[4] & 0xFFFFu) | (c[5] << 16);
        o.w = (c[6] & 0xFFFFu) | (c[7] << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(p16 + r_lo * 256 + 8 * k));
      } else {
        u32x2 o;
        o.x = (c[0] & 0xFFu) | ((c[1] & 0xFFu) << 8) | ((c[2] & 0xFFu) << 16) | ((c[3] & 0xFFu) << 24);
        o.y = (c[4] & 0xFFu) | ((c[5] & 0xFFu) << 8) | ((c[6] & 0xFFu) << 16) | ((c[7] & 0xFFu) << 24);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(ws + r_lo * 256 + 8 * k));
      }
      if (wide_hi) {
        u32x4 o;
        o.x = (c[0] >> 16) | (c[1] & 0xFFFF0000u);
        o.y = (c[2] >> 16) | (c[3] & 0xFFFF0000u);
        o.z = (c[4] >> 16) | (c[5] & 0xFFFF0000u);
        o.w = (c[6] >> 16) | (c[7] & 0xFFFF0000u);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(p16 + r_hi * 256 + 8 * k));
      } else {
        u32x2 o;
        o.x = ((c[0] >> 16) & 0xFFu) | (((c[1] >> 16) & 0xFFu) << 8) | (((c[2] >> 16) & 0xFFu) << 16) |
              ((c[3] >> 16) << 24);
        o.y = ((c[4] >> 16) & 0xFFu) | (((c[5] >> 16) & 0xFFu) << 8) | (((c[6] >> 16) & 0xFFu) << 16) |
              ((c[7] >> 16) << 24);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(ws + r_hi * 256 + 8 * k));
      }
      if (k == 0) {
        flag[r_lo] = wide_lo ? 1 : 0;
        flag[r_hi] = wide_hi ? 1 : 0;
      }
    }
  } else if constexpr (LO) {
    // low-byte counts spread over the bins: one 32-bit atomic per counter
    hist16_flush<E>(lds_hist, hist + int64_t(layer) * E * 256, tid, kRHThreads, g);
  } else {
    hist16_flush_pairs<E>(lds_hist, hist + int64_t(layer) * E * 256, tid, kRHThreads, g);
  }
}

template <int E>
static int launch_rh(bool lo, const float* s, const float* alpha, int L, int64_t N,
                     const int32_t* sel_hi, int32_t* hist, hipStream_t st) {
  const RowSplit sp = split_rows(L, N, RHShape<E>::STEP, QB_RH_MAXROWS);
  if (lo)
    hipLaunchKernelGGL((k_radix_hist<E, true, false>), dim3(unsigned(sp.blocks)), dim3(kRHThreads), 0, st,
                       s, alpha, N, sp.wg_per_layer, sel_hi, hist, nullptr, int64_t(0), int64_t(0));
  else
    hipLaunchKernelGGL((k_radix_hist<E, false, false>), dim3(unsigned(sp.blocks)), dim3(kRHThreads), 0, st,
                       s, alpha, N, sp.wg_per_layer, sel_hi, hist, nullptr, int64_t(0), int64_t(0));
  return int(hipGetLastError());
}

template <int E>
static int launch_rh_ws(const float* s, const float* alpha, int L, int64_t N, const int32_t* sel_hi,
                        uint8_t* ws, hipStream_t st) {
  const RowSplit sp = split_rows(L, N, RHShape<E>::STEP, QB_RH_MAXROWS);
  const LoWs lay = lo_ws_layout(L, E, sp.wg_per_layer);
  hipLaunchKernelGGL((k_radix_hist<E, true, true>), dim3(unsigned(sp.blocks)), dim3(kRHThreads), 0, st, s,
                     alpha, N, sp.wg_per_layer, sel_hi, nullptr, ws, lay.flag, lay.p16);
  return int(hipGetLastError());
}

int radix_wg_per_layer(int L, int64_t N, int E) {
  switch (E) {
    case 16: return split_rows(L, N, RHShape<16>::STEP, QB_RH_MAXROWS).wg_per_layer;
    case 32: return split_rows(L, N, RHShape<32>::STEP, QB_RH_MAXROWS).wg_per_layer;
    case 64: return split_rows(L, N, RHShape<64>::STEP, QB_RH_MAXROWS).wg_per_layer;
    case 128: return split_rows(L, N, RHShape<128>::STEP, QB_RH_MAXROWS).wg_per_layer;
    case 256: return split_rows(L, N, RHShape<256>::STEP, QB_RH_MAXROWS).wg_per_layer;
  }
  return 0;
}

int launch_radix_hist_lo_ws(const float* s, const float* alpha, int L, int64_t N, int E,
                            const int32_t* sel_hi, uint8_t* ws, hipStream_t st) {
  switch (E) {
    case 16: return launch_rh_ws<16>(s, alpha, L, N, sel_hi, ws, st);
    case 32: return launch_rh_ws<32>(s, alpha, L, N, sel_hi, ws, st);
    case 64: return launch_rh_ws<64>(s, alpha, L, N, sel_hi, ws, st);
    case 128: return launch_rh_ws<128>(s, alpha, L, N, sel_hi, ws, st);
    case 256: return launch_rh_ws<256>(s, alpha, L, N, sel_hi, ws, st);
  }
  return int(hipErrorInvalidValue);
}

int launch_radix_hist(bool lo, const float* s, const float* alpha, int L, int64_t N, int E,
                      const int32_t* sel_hi, int32_t* hist, hipStream_t st) {
  switch (E) {
    case 16: return launch_rh<16>(lo, s, alpha, L, N, sel_hi, hist, st);
    case 32: return launch_rh<32>(lo, s, alpha, L, N, sel_hi, hist, st);
    case 64: return launch_rh<64>(lo, s, alpha, L, N, sel_hi, hist, st);
    case 128: return launch_rh<128>(lo, s, alpha, L, N, sel_hi, hist, st);
    case 256: return launch_rh<256>(lo, s, alpha, L, N, sel_hi, hist, st);
  }
  return int(hipErrorInvalidValue);
}

// ---------------------------------------------------------------------------
// Keys of every margin, token-major u16 [L][N][E] (same layout as s).
constexpr int kMKThreads = 256;

__global__ __launch_bounds__(kMKThreads) void k_margin_keys(const float* __restrict__ s,
                                                            const float* __restrict__ alpha,
                                                            int64_t N, int E,
                                                            uint16_t* __restrict__ keys) {
  const int64_t total4 = N * E / 4;  // float4 groups of one layer
  const int layer = blockIdx.y;
  s += int64_t(layer) * N * E;
  alpha += int64_t(layer) * N;
  keys += int64_t(layer) * N * E;
  const int64_t stride = int64_t(gridDim.x) * kMKThreads;
  for (int64_t i = int64_t(blockIdx.x) * kMKThreads + threadIdx.x; i < total4; i += stride) {
    const float4 x = ld4(s + 4 * i);
    const float a = alpha[(4 * i) / E];
    const uint32_t k01 = key2(bf16x2_rne(a - x.x, a - x.y));
    const uint32_t k23 = key2(bf16x2_rne(a - x.z, a - x.w));
    *reinterpret_cast<uint2*>(keys + 4 * i) = make_uint2(k01, k23);
  }
}

int launch_margin_keys(const float* s, const float* alpha, int L, int64_t N, int E, uint16_t* keys,
                       hipStream_t st) {
  const int64_t total4 = N * E / 4;
  const int64_t bx = std::min<int64_t>(int64_t(device_cu_count()) * 8,
                                       std::max<int64_t>(1, (total4 + kMKThreads - 1) / kMKThreads));
  hipLaunchKernelGGL(k_margin_keys, dim3(unsigned(bx), unsigned(L)), dim3(kMKThreads), 0, st, s, alpha,
                     N, E, keys);
  return int(hipGetLastError());
}

}  // namespace qbk
