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

// 1: each workgroup walks its trips from the last to the first.  Pass 1
// reads the scores in ascending row order, so the rows it read last (still
// in the 256 MB memory-side Infinity Cache) are the ones this pass reads
// first, and the next pass 1 starts on the rows this pass read last.  EQB
// step at E = 256 (graph of 20 steps): 381-386 -> 371-375 us at 1M rows,
// 216-217 -> 204 us at 512K; no change at 256K rows or 48 x 256K.
#ifndef QB_RH_REVERSE
#define QB_RH_REVERSE 1
#endif
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
//
// LD (low-byte pass only): the top-K loads of s + b are counted on the way
// ("[Dev] Add global-batch quantile balancing", section "Quantile
// estimator": the K largest of s + b route a token; "Exact Quantile
// Balancing and Load-Error Injection for Mixture-of-Experts", LEI
// paragraph: the per-expert loads behind the relative load errors), with
// alpha from pass 1: a token's members are its v = s + b > alpha plus, when
// alpha's value is tied, the lowest-index elements equal to alpha up to K.
// Here a lane's four experts are fixed for the whole kernel, so their bias
// sits in four registers and the lane counts their members in four register
// counters; a row's count above alpha and its tie ranks come from ballots
// over the lanes holding the row.  LD = 1: load[l][e] += counts, added once
// per workgroup; LD = 2: also load_mb[l][c][e] for each n_mb-row
// microbatch c (n_mb a multiple of the trip), the counts of each trip summed
// in LDS and added to its microbatch's row.  No LDS atomic per element and
// no bias reads from LDS: the standalone pass 1 pays for both.
template <int E, bool LO, bool WS, int LD = 0, bool ST = false>
__global__ __launch_bounds__(kRHThreads) void k_radix_hist(
    const float* __restrict__ s, const float* __restrict__ alpha, int64_t N, int wg_per_layer,
    const int32_t* __restrict__ sel_hi, int32_t* __restrict__ hist, uint8_t* __restrict__ ws,
    int64_t ws_flag, int64_t ws_p16, const float* __restrict__ bias, int K, int32_t* __restrict__ load,
    int32_t* __restrict__ load_mb, int64_t n_mb) {
  using S = RHShape<E>;
  static_assert(LD == 0 || LO, "loads are counted in the low-byte pass");
  __shared__ uint32_t lds_hist[(E / 2) * 256];
  // LD == 1: the workgroup's totals; LD == 2: two trip buffers, then the totals
  constexpr int kLdsLoad = LD == 2 ? 3 * E : (LD == 1 ? E : 1);
  __shared__ int32_t lds_load[kLdsLoad];
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
  // load counting: the bias of the lane's four experts and its counters
  float bq[4] = {0.f, 0.f, 0.f, 0.f};
  int cnt[4] = {0, 0, 0, 0};  // this trip's (LD == 2) or all trips' (LD == 1) members
  int tot[4] = {0, 0, 0, 0};  // LD == 2: all trips' members
  if constexpr (LD > 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bq[c] = bias[int64_t(layer) * E + 4 * quad + c];
      asm volatile("" : "+v"(bq[c]));
    }
    for (int j = tid; j < kLdsLoad; j += kRHThreads) lds_load[j] = 0;
    if constexpr (LD == 2) load_mb += int64_t(layer) * (N / n_mb) * E;
    load += int64_t(layer) * E;
  }
  // lanes of this lane's row (QPR lanes) and those of them below this lane
  const uint64_t seg = S::QPR >= 64 ? ~0ull : (((1ull << S::QPR) - 1ull) << (rsub * S::QPR));
  const uint64_t below = seg & ((1ull << lane) - 1ull);
  __syncthreads();

  // Full trips (every row < N): addresses from the wave-uniform row base
  // with 32-bit lane offsets, no clamps and no per-row tests, so the loop
  // body is straight-line and each set's loads are waited for one by one.
  auto load_full = [&](int64_t base, float4 (&x)[S::U], float (&a)[S::U]) {
    const float* sw = s + base * E;
    const float* aw = alpha + base;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      x[u] = (ST ? ld4_nt : ld4)(sw + uint32_t((u * S::RPI + rsub) * E + 4 * quad));
      a[u] = aw[u * S::RPI + rsub];
    }
  };
  auto count_load = [&](const float4& x, float a, bool valid) {
    const float v0 = x.x + bq[0], v1 = x.y + bq[1], v2 = x.z + bq[2], v3 = x.w + bq[3];
    const bool g0 = valid && v0 > a, g1 = valid && v1 > a, g2 = valid && v2 > a, g3 = valid && v3 > a;
    const uint64_t b0 = __ballot(g0), b1 = __ballot(g1), b2 = __ballot(g2), b3 = __ballot(g3);
    const int need = K - (__popcll(b0 & seg) + __popcll(b1 & seg) + __popcll(b2 & seg) + __popcll(b3 & seg));
    int m0 = g0, m1 = g1, m2 = g2, m3 = g3;
    if (__ballot(valid && need > 0) != 0) {  // a tie at alpha in some row of this instruction
      const bool e0 = valid && v0 == a, e1 = valid && v1 == a, e2 = valid && v2 == a, e3 = valid && v3 == a;
      const uint64_t q0 = __ballot(e0), q1 = __ballot(e1), q2 = __ballot(e2), q3 = __ballot(e3);
      // equal elements of the row with a lower expert index (4 quad + c)
      const int r0 = __popcll(q0 & below) + __popcll(q1 & below) + __popcll(q2 & below) + __popcll(q3 & below);
      m0 |= e0 && r0 < need;
      m1 |= e1 && r0 + e0 < need;
      m2 |= e2 && r0 + e0 + e1 < need;
      m3 |= e3 && r0 + e0 + e1 + e2 < need;
    }
    cnt[0] += m0;
    cnt[1] += m1;
    cnt[2] += m2;
    cnt[3] += m3;
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
  auto trip_of = [&](int64_t k) -> int64_t { return QB_RH_REVERSE && k < nF ? nF - 1 - k : k; };
  auto trip_base = [&](int64_t k) {
    return (int64_t(g) + trip_of(k) * wg_per_layer) * S::STEP + int64_t(wave) * S::RPW;
  };
  const bool early = wave >= kRHWaves / 2;
  // LD == 2: each lane adds its counts of trip k into LDS buffer k & 1 at
  // the end of the trip; wave 0 adds that buffer to trip k's microbatch row
  // and clears it after the barrier that opens trip k + 1, which every wave
  // reaches after its adds, and before the barrier that opens trip k + 2,
  // after which the waves add into it again.  The bare barriers order no
  // LDS access by themselves: each wave first waits for its own LDS
  // operations (lgkmcnt 0; the row loads stay in flight).
  auto mb_flush = [&](int64_t kt) {  // wave 0: trip number kt of this workgroup
    const int64_t mb = ((int64_t(g) + trip_of(kt) * wg_per_layer) * S::STEP) / n_mb;
    int32_t* buf = lds_load + (kt & 1) * E;
    for (int j = lane; j < E; j += kWave) {
      const int32_t v = buf[j];
      if (v) {
        atomicAdd(load_mb + mb * E + j, v);
        buf[j] = 0;
      }
    }
  };
  auto trip_loads_done = [&](int64_t kt) {
    if constexpr (LD == 2) {
      int32_t* buf = lds_load + (kt & 1) * E;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (cnt[c]) atomicAdd(&buf[4 * quad + c], cnt[c]);
        tot[c] += cnt[c];
        cnt[c] = 0;
      }
    }
  };
  auto lds_wait_barrier = [&]() {
    if constexpr (LD == 2) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
  };
  float4 x[S::U];
  float a[S::U];
  for (int64_t k = 0; k < nF; ++k) {
    if (early) {
      load_full(trip_base(k), x, a);
      lds_wait_barrier();
    } else {
      lds_wait_barrier();
      load_full(trip_base(k), x, a);
    }
    if constexpr (LD == 2) {
      if (k > 0 && wave == 0) mb_flush(k - 1);
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      count1(x[u], a[u]);
      if constexpr (LD > 0) count_load(x[u], a[u], true);
    }
    trip_loads_done(k);
  }
  if constexpr (LD == 2) {
    // every wave's adds of trip nF - 1 are done, and wave 0's clearing of
    // buffer nF & 1 (trip nF - 2) before the partial trip adds into it
    lds_wait_barrier();
    if (nF > 0 && wave == 0) mb_flush(nF - 1);
  }
  const int64_t base = trip_base(nF);
  const bool partial = base < N;  // wave 0 has a partial trip if any wave has
  if (partial) {
    // the partial trip: rows clamped to N - 1 for the loads, not counted
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      int64_t row = base + u * S::RPI + rsub;
      row = row < N ? row : N - 1;
      x[u] = (ST ? ld4_nt : ld4)(s + row * E + 4 * quad);
      a[u] = alpha[row];
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u)
      if (base + u * S::RPI + rsub < N) count1(x[u], a[u]);
  }
  if constexpr (LD > 0) {
    // rows past N count nothing (valid = false), and the ballots see every
    // lane of the wave
    if (__builtin_amdgcn_readfirstlane(int(partial))) {
#pragma unroll
      for (int u = 0; u < S::U; ++u) count_load(x[u], a[u], base + u * S::RPI + rsub < N);
    }
    if constexpr (LD == 2) {
      if (partial) trip_loads_done(nF);
    }
  }
  if constexpr (LD > 0) {
    // the workgroup's totals, through LDS, then one atomic per expert
    int32_t* lt = lds_load + (LD == 2 ? 2 * E : 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int v = LD == 2 ? tot[c] : cnt[c];
      if (v) atomicAdd(&lt[4 * quad + c], v);
    }
  }
  __syncthreads();
  if constexpr (LD > 0) {
    if constexpr (LD == 2) {
      if (partial && wave == 0) mb_flush(nF);
    }
    const int32_t* lt = lds_load + (LD == 2 ? 2 * E : 0);
    for (int j = tid; j < E; j += kRHThreads)
      if (lt[j]) atomicAdd(load + j, lt[j]);
  }
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
                       s, alpha, N, sp.wg_per_layer, sel_hi, hist, nullptr, int64_t(0), int64_t(0), nullptr, 0,
                       nullptr, nullptr, int64_t(1));
  else
    hipLaunchKernelGGL((k_radix_hist<E, false, false>), dim3(unsigned(sp.blocks)), dim3(kRHThreads), 0, st,
                       s, alpha, N, sp.wg_per_layer, sel_hi, hist, nullptr, int64_t(0), int64_t(0), nullptr, 0,
                       nullptr, nullptr, int64_t(1));
  return int(hipGetLastError());
}

template <int E>
static int launch_rh_ws(const float* s, const float* alpha, int L, int64_t N, const int32_t* sel_hi,
                        uint8_t* ws, hipStream_t st, const float* b = nullptr, int K = 0, int32_t* load = nullptr,
                        int64_t n_mb = 1, int32_t* load_mb = nullptr) {
  const RowSplit sp = split_rows(L, N, RHShape<E>::STEP, QB_RH_MAXROWS);
  const LoWs lay = lo_ws_layout(L, E, sp.wg_per_layer);
  const dim3 grid(unsigned(sp.blocks)), block(kRHThreads);
  // layers far larger than the Infinity Cache are read with non-temporal
  // loads (stream_pass); rows of at least 128 bytes, so that every load
  // instruction takes whole lines
  if constexpr (E >= 32) {
    if (stream_pass(L, N, E)) {
      if (load && load_mb)
        hipLaunchKernelGGL((k_radix_hist<E, true, true, 2, true>), grid, block, 0, st, s, alpha, N, sp.wg_per_layer,
                           sel_hi, nullptr, ws, lay.flag, lay.p16, b, K, load, load_mb, n_mb);
      else if (load)
        hipLaunchKernelGGL((k_radix_hist<E, true, true, 1, true>), grid, block, 0, st, s, alpha, N, sp.wg_per_layer,
                           sel_hi, nullptr, ws, lay.flag, lay.p16, b, K, load, nullptr, int64_t(1));
      else
        hipLaunchKernelGGL((k_radix_hist<E, true, true, 0, true>), grid, block, 0, st, s, alpha, N, sp.wg_per_layer,
                           sel_hi, nullptr, ws, lay.flag, lay.p16, nullptr, 0, nullptr, nullptr, int64_t(1));
      return int(hipGetLastError());
    }
  }
  if (load && load_mb)
    hipLaunchKernelGGL((k_radix_hist<E, true, true, 2>), grid, block, 0, st, s, alpha, N, sp.wg_per_layer, sel_hi,
                       nullptr, ws, lay.flag, lay.p16, b, K, load, load_mb, n_mb);
  else if (load)
    hipLaunchKernelGGL((k_radix_hist<E, true, true, 1>), grid, block, 0, st, s, alpha, N, sp.wg_per_layer, sel_hi,
                       nullptr, ws, lay.flag, lay.p16, b, K, load, nullptr, int64_t(1));
  else
    hipLaunchKernelGGL((k_radix_hist<E, true, true, 0>), grid, block, 0, st, s, alpha, N, sp.wg_per_layer, sel_hi,
                       nullptr, ws, lay.flag, lay.p16, nullptr, 0, nullptr, nullptr, int64_t(1));
  return int(hipGetLastError());
}

// Trip size of the low-byte pass, rows: microbatches of the load counting
// must be a multiple of it.
int radix_lo_trip_rows(int E) {
  switch (E) {
    case 16: return RHShape<16>::STEP;
    case 32: return RHShape<32>::STEP;
    case 64: return RHShape<64>::STEP;
    case 128: return RHShape<128>::STEP;
    case 256: return RHShape<256>::STEP;
  }
  return 0;
}

int launch_radix_hist_lo_ws_loads(const float* s, const float* alpha, int L, int64_t N, int E,
                                  const int32_t* sel_hi, uint8_t* ws, const float* b, int K, int32_t* load,
                                  int64_t n_mb, int32_t* load_mb, hipStream_t st) {
  switch (E) {
    case 16: return launch_rh_ws<16>(s, alpha, L, N, sel_hi, ws, st, b, K, load, n_mb, load_mb);
    case 32: return launch_rh_ws<32>(s, alpha, L, N, sel_hi, ws, st, b, K, load, n_mb, load_mb);
    case 64: return launch_rh_ws<64>(s, alpha, L, N, sel_hi, ws, st, b, K, load, n_mb, load_mb);
    case 128: return launch_rh_ws<128>(s, alpha, L, N, sel_hi, ws, st, b, K, load, n_mb, load_mb);
    case 256: return launch_rh_ws<256>(s, alpha, L, N, sel_hi, ws, st, b, K, load, n_mb, load_mb);
  }
  return int(hipErrorInvalidValue);
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
