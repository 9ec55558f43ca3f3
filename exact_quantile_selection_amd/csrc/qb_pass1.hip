// qb_pass1.hip -- first pass over the score matrix: per-token top-(K+1) of
// s + b (alpha), optional top-K load counts, and the fused high-byte
// histogram of the bf16 margin keys.
//
// Method: "[Dev] Add global-batch quantile balancing" (Megatron-LM PR #6637),
// section "Quantile estimator" (alpha = (k+1)-th largest of s + b, margin
// r = alpha - s); "Exact Quantile Balancing and Load-Error Injection for
// Mixture-of-Experts" (summary page), EQB paragraph (first radix pass: 256-bin
// histogram of the high byte of the bf16 margins).
//
// Layout on gfx950: a row of E fp32 scores is split over 4 lanes, each
// holding V = E/4 scores in registers (V/4 float4 loads), so a load
// instruction covers 16 rows; a wave trip takes 16 / (V/4) such row groups
// (64 scores per lane).  The lanes of one row read 64 contiguous bytes per
// load; the starting column block is rotated by the row index so that, in
// every later instruction, the lanes of the wave touch distinct experts
// (distinct LDS banks for the histogram atomics, distinct bias entries) as
// far as E allows.  The high-byte pass without loads rotates whole 128-byte
// lines instead for E >= 64 (two consecutive loads of a lane take the two
// halves of one line), and over layers of 768 MiB or more at E = 256 it
// splits a row over 8 lanes and reads it with non-temporal loads.
//   * top-(K+1): per-lane insertion with v_med3_f32 (one op per list slot),
//     then DPP merges across the row's lanes (bitonic), the last merge only
//     producing the minimum of the merged top list, which is alpha.
//   * histogram: keys of both halves of a packed bf16 pair are made in three
//     integer ops; counters are 16-bit pairs in LDS (E*512 bytes), flushed to
//     the global int32 histogram once per workgroup (<= 65535 rows each).
//   * full-key mode (HM = 2): instead, every 16-bit key is counted into a
//     global [E][65536] int32 histogram with one device atomic per element
//     -- the one-pass alternative the EQB paragraph compares the two byte
//     histograms against (128x their memory); kept for that comparison.
//   * work split: a workgroup trip is 16 waves x (64/LPR) rows; trips are
//     block-cyclic over the workgroups, so the workgroups in flight read
//     neighbouring rows (all HBM channels busy).  A full trip addresses its
//     rows from a wave-uniform base with 32-bit lane offsets; only the last,
//     partial trip clamps rows.
#include "qb_device.hpp"
#include "qb_internal.hpp"

// Pass 1 without loads refills each score slot with the next trip's row as
// soon as the slot's key is counted (1; 0: the whole trip loaded at once by
// half of the waves before the trip's barrier and half after it; 2: rolling
// without the barrier).
#ifndef QB_P1_ROLL
#define QB_P1_ROLL 1
#endif
// The rolling path issues its first trip's loads before it clears the LDS
// table (65,536 x 256: EQB step 54.1-54.2 against 54.6-54.8 us; no change
// at 262,144 and 1M tokens).
#ifndef QB_P1_EARLY
#define QB_P1_EARLY 1
#endif

// Rows per workgroup at most (16-bit LDS counters hold 65535); smaller
// values give more, shorter-lived workgroups.
#ifndef QB_P1_MAXROWS
#define QB_P1_MAXROWS 65535
#endif

namespace qbk {

#ifndef QB_P1_WAVES
#define QB_P1_WAVES 16
#endif
// QB_P1_WAVES waves per workgroup (<= 128 VGPRs each) for lists of up to 8,
// also with load counting (the count runs after the histogram, from the raw
// scores and bias values re-read from LDS, so it fits); lists longer than 8
// keep more state per lane and run 8 waves (<= 256 VGPRs each), and the
// per-microbatch count 12 (<= 168).  Measured on one MI355X, alpha + loads +
// high-byte histogram at 1,048,576 x 256: 245 us with 8 waves, 229 with 12,
// 224 with 16; with microbatch loads 222, 216 and 225 us.
template <bool LOAD, int P, bool MB = false>
constexpr int p1_waves() { return P > 8 ? 8 : (MB ? 12 : QB_P1_WAVES); }

// Every E splits a row over 4 lanes, so the lanes of one row read E bytes
// contiguously (64 B at E = 16, 1 KiB at E = 256) and a load instruction
// covers 16 rows; narrower rows give each lane several row groups per trip
// (U), so that every lane holds 64 scores per trip at every E.  (One lane
// per row for E <= 64 made each load instruction touch 64 rows 16 bytes at
// a time: 1 GiB of scores at E = 64 took 247 us in pass 1 against 190 at
// E = 256.)
template <int E, int LPR_ = 4>
struct P1Shape {
  static constexpr int LPR = LPR_;           // lanes per row
  static constexpr int V = E / LPR;          // scores per lane and row
  static constexpr int F4 = V / 4;           // float4 loads per lane and row
  static constexpr int RPW = kWave / LPR;    // rows per row group of a wave
  static constexpr int U = 16 / F4;          // row groups per wave trip
  static constexpr int WROWS = RPW * U;      // rows per wave trip
  static constexpr int HDW = (E / 2) * 256;
  // copies of the high-byte table (128 KiB in all): the 16 rows of a load
  // instruction share E/4 expert groups, and with fewer than 256 experts
  // lanes of different rows would add into the same hot counters; row rho
  // of the group counts into copy rho % NC.
  static constexpr int NC = 256 / E;
  static_assert(E % 16 == 0 && E <= 256, "experts");
  static_assert((F4 & (F4 - 1)) == 0, "power-of-two loads per lane");
};

// Paired column order for the high-byte pass without loads (1): slots 2i
// and 2i + 1 of a lane read the two halves of one 128-byte line of its row,
// the line rotated by the row.  A read probe over 1 GiB of 1 KiB rows, 4
// lanes per row: 166 us against 177 us for the plain rotation.  Pass 1 over
// 1 GiB of scores (events, two runs each): E = 64 208-209 against 223-225 us,
// E = 128 210-215 against 214-219 us, unchanged at 262,144 x 256; the
// alpha-only pass gains nothing from it (the 65,536-token K3 step 56 against
// 55 us), and at E = 32 (one line per row: no rotation left) 224 against
// 215 us, so neither takes it.
#ifndef QB_P1_PAIR
#define QB_P1_PAIR 1
#endif

// The column block (of LPR float4s) that a lane group reads in slot t of its
// row; rot is the row index within the load instruction.  Plain: block
// (t + rot) mod F4, so the rows of one instruction cover distinct columns as
// far as E allows.  PAIR (4 lanes per row, at least two lines per row): the
// lines are rotated instead, block 2 ((t / 2 + rot) mod F4/2) + t mod 2.
template <class S, bool PAIR>
__device__ __forceinline__ int p1_blk(int t, int rot) {
  if constexpr (PAIR && S::LPR == 4 && S::F4 >= 4) return ((((t >> 1) + rot) & (S::F4 / 2 - 1)) << 1) | (t & 1);
  return (t + rot) & (S::F4 - 1);
}

// The high-byte table copy of row rho of a load instruction.  In the paired
// order rows rho and rho' of one instruction read the same columns when
// rho = rho' mod F4/2, and rho / (F4/2) mod NC spreads them over the copies.
// In the plain order (rho = rho' mod F4) rho mod NC lets some of them share
// a copy for 32 <= E <= 128; copies chosen by rho / F4 mod NC, which never
// share, measured the same (one GiB of scores at E = 32: 212-215 us).
template <class S, bool PAIR = false>
__device__ __forceinline__ int p1_copy(int rho) {
  if constexpr (PAIR && S::LPR == 4 && S::F4 >= 4) return (rho / (S::F4 / 2)) % S::NC;
  return rho % S::NC;
}


__device__ __forceinline__ uint64_t low_bits(int n) {
  return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
}

// Rotates the low V bits of m left by n (0 <= n < V).
template <int V>
__device__ __forceinline__ uint64_t rotl_v(uint64_t m, int n) {
  if constexpr (V == 64) {
    return n == 0 ? m : (m << n) | (m >> (64 - n));
  } else {
    constexpr uint64_t kMask = (1ull << V) - 1ull;
    return n == 0 ? m : (((m << n) | (m >> (V - n))) & kMask);
  }
}

// Top-K membership of this lane's scores for one row, added to the LDS load
// counters.  Members are v > alpha plus, when alpha's value occurs more than
// once, the lowest-index elements equal to alpha up to K in total.  A lane's
// element (u, c) has expert j = 4*(LPR*u + ql) + c and mask bit 4u + c, so
// bit order is j order within a lane.  The masks are first built in load
// order (bit 4t + c, constant positions) and then rotated by the lane's
// column rotation; the counters take one LDS atomic per member.  Only the
// "greater than alpha" mask is built for every row: fewer than K elements
// exceed alpha only when alpha's value is tied, and then the whole wave
// builds the "equal to alpha" masks and ranks the tied elements.
template <int E, int P>
__device__ __forceinline__ void count_loads(const float4 (&x)[P1Shape<E>::F4], const float* lds_b,
                                            int rho, int ql, float a, int K, bool valid,
                                            int32_t* lds_load) {
  using S = P1Shape<E>;
  // An opaque copy of the rotation: the compiler cannot tell that these bias
  // reads repeat the top-(K+1) loop's, so it re-reads them from LDS instead
  // of keeping that loop's bias values live until here.
  asm volatile("" : "+v"(rho));
  uint64_t gt_t = 0;
#pragma unroll
  for (int t = 0; t < S::F4; ++t) {
    const int quad = S::LPR * ((t + rho) & (S::F4 - 1)) + ql;
    const float4 bb = *reinterpret_cast<const float4*>(&lds_b[4 * quad]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float v = comp(x[t], c) + comp(bb, c);
      gt_t |= v > a ? 1ull << (4 * t + c) : 0ull;
    }
  }
  const int rot = 4 * (rho & (S::F4 - 1));
  uint64_t mem = rotl_v<S::V>(gt_t, rot);
  int G = __popcll(gt_t);
  if constexpr (S::LPR >= 2) G += quad_mov_i<kQuadXor1>(G);
  if constexpr (S::LPR == 4) G += quad_mov_i<kQuadXor2>(G);
  const int need = K - G;  // equal-to-alpha elements that still belong to the top K
  if (__ballot(valid && need > 0) != 0) {  // wave-uniform: every lane takes part
    uint64_t eq_t = 0;
#pragma unroll
    for (int t = 0; t < S::F4; ++t) {
      const int quad = S::LPR * ((t + rho) & (S::F4 - 1)) + ql;
      const float4 bb = *reinterpret_cast<const float4*>(&lds_b[4 * quad]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = comp(x[t], c) + comp(bb, c);
        eq_t |= v == a ? 1ull << (4 * t + c) : 0ull;
      }
    }
    const uint64_t eq = rotl_v<S::V>(eq_t, rot);
    // equal-to-alpha masks of the row's lanes
    uint64_t M[S::LPR];
#pragma unroll
    for (int q2 = 0; q2 < S::LPR; ++q2) {
      const int src = rho * S::LPR + q2;
      const uint32_t lo = __shfl(uint32_t(eq), src);
      const uint32_t hi = __shfl(uint32_t(eq >> 32), src);
      M[q2] = (uint64_t(hi) << 32) | lo;
    }
    if (valid && need > 0) {
      // an element equal to alpha is a member when fewer than `need` equal
      // elements of the row precede it in expert order
      uint64_t e = eq;
      while (e) {
        const int bit = __builtin_ctzll(e);
        e &= e - 1;
        const int u = bit >> 2, c = bit & 3;
        int r = 0;
#pragma unroll
        for (int q2 = 0; q2 < S::LPR; ++q2) {
          const int nb = q2 < ql ? 4 * (u + 1) : (q2 > ql ? 4 * u : 4 * u + c);
          r += __popcll(M[q2] & low_bits(nb));
        }
        if (r < need) mem |= 1ull << bit;
      }
    }
  }
  if (!valid) return;
  while (mem) {
    const int bit = __builtin_ctzll(mem);
    mem &= mem - 1;
    const int e = 4 * (S::LPR * (bit >> 2) + ql) + (bit & 3);
    atomicAdd(&lds_load[e], 1);
  }
}

// Loads one trip's rows (this lane's V scores of row base + rho) into x.
// `base` is wave-uniform: a full trip addresses its rows from a uniform base
// pointer with 32-bit lane offsets; a partial last trip clamps the row.
template <int E, int LPR = 4, bool STREAM = false, bool PAIR = false>
__device__ __forceinline__ void p1_load(const float* s, int64_t base, int64_t N, int rho, int ql,
                                        float4 (&x)[(P1Shape<E, LPR>::F4)]) {
  using S = P1Shape<E, LPR>;
  // The per-slot bias values, addresses and swizzles are loop-invariant;
  // kept invariant they would be hoisted out of the row loop and occupy ~100
  // VGPRs.  An opaque copy of the rotation makes them cheap per-trip work.
  int rot = rho;
  asm volatile("" : "+v"(rot));
  if (base + S::RPW <= N) {
    const float* ws = s + base * E;
    const uint32_t lane_off = uint32_t(rho * E + 4 * ql);
#pragma unroll
    for (int t = 0; t < S::F4; ++t)
      x[t] = (STREAM ? ld4_nt : ld4)(ws + (lane_off + uint32_t(4 * S::LPR * p1_blk<S, PAIR>(t, rot))));
  } else {
    const int64_t row = base + rho;
    const float* src = s + (row < N ? row : N - 1) * E;
#pragma unroll
    for (int t = 0; t < S::F4; ++t) {
      const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
      x[t] = (STREAM ? ld4_nt : ld4)(src + 4 * quad);
    }
  }
}

// p1_rows without loads (HM = 1) that refills each slot of x with the next
// trip's scores (rows nbase + rho) as soon as the slot's last use, its key,
// is done: the next trip streams in while this one is counted.
template <int E, int P, int LPR = 4, bool STREAM = false, bool PAIR = false>
__device__ __forceinline__ void p1_rows_roll(float4 (&x)[(P1Shape<E, LPR>::F4)], const float* s, int64_t base,
                                             int64_t nbase, bool more, int64_t N, int rho, int ql,
                                             const float* lds_b, uint32_t* lds_hist, float* alpha) {
  using S = P1Shape<E, LPR>;
  const int64_t row = base + rho;
  const bool valid = row < N;
  int rot = rho;
  asm volatile("" : "+v"(rot));
  float top[P];
#pragma unroll
  for (int k = 0; k < P; ++k) top[k] = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < S::F4; ++t) {
    const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
    const float4 bb = *reinterpret_cast<const float4*>(&lds_b[4 * quad]);
    top_insert<P>(top, x[t].x + bb.x);
    top_insert<P>(top, x[t].y + bb.y);
    top_insert<P>(top, x[t].z + bb.z);
    top_insert<P>(top, x[t].w + bb.w);
  }
  float a;
  if constexpr (S::LPR == 1) {
    a = top[P - 1];
  } else if constexpr (S::LPR == 2) {
    a = top_merge_last<P, kQuadXor1>(top);
  } else if constexpr (S::LPR == 4) {
    top_merge<P, kQuadXor1>(top);
    a = top_merge_last<P, kQuadXor2>(top);
  } else {
    top_merge<P, kQuadXor1>(top);
    top_merge<P, kQuadXor2>(top);
    a = top_merge_last<P, kHalfMirror>(top);
  }
  if (valid && ql == 0) __builtin_nontemporal_store(a, alpha + row);
  uint32_t* h = lds_hist + (S::NC > 1 ? p1_copy<S, PAIR>(rho) * S::HDW : 0);
  if (more) {
    const int64_t nrow = nbase + rho;
    const float* np = s + (nrow < N ? nrow : N - 1) * E;
#pragma unroll
    for (int t = 0; t < S::F4; ++t) {
      const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
      if (valid) {
        const uint32_t swz = hist16_swizzle2(quad);
        hist16_add_hi(h, quad, 0, key2(bf16x2_rne(a - x[t].x, a - x[t].y)) ^ swz);
        hist16_add_hi(h, quad, 2, key2(bf16x2_rne(a - x[t].z, a - x[t].w)) ^ swz);
      }
      x[t] = (STREAM ? ld4_nt : ld4)(np + 4 * quad);
    }
  } else if (valid) {
#pragma unroll
    for (int t = 0; t < S::F4; ++t) {
      const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
      const uint32_t swz = hist16_swizzle2(quad);
      hist16_add_hi(h, quad, 0, key2(bf16x2_rne(a - x[t].x, a - x[t].y)) ^ swz);
      hist16_add_hi(h, quad, 2, key2(bf16x2_rne(a - x[t].z, a - x[t].w)) ^ swz);
    }
  }
}

// alpha, loads and the high-byte histogram of one trip's rows.
template <int E, int P, int HM, bool LOAD, bool PAIR = false>
__device__ __forceinline__ void p1_rows(const float4 (&x)[P1Shape<E>::F4], int64_t base, int64_t N,
                                        int rho, int ql, int lane, int K, const float* lds_b,
                                        uint32_t* lds_hist, int32_t* lds_load, float* alpha,
                                        int32_t* ghist) {
  using S = P1Shape<E>;
  static_assert(!(PAIR && LOAD), "the load count assumes the plain column order");
  const int64_t row = base + rho;
  const bool valid = row < N;
  int rot = rho;
  asm volatile("" : "+v"(rot));
  float top[P];
#pragma unroll
  for (int k = 0; k < P; ++k) top[k] = -__builtin_inff();
#pragma unroll
  for (int t = 0; t < S::F4; ++t) {
    const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
    const float4 bb = *reinterpret_cast<const float4*>(&lds_b[4 * quad]);
    top_insert<P>(top, x[t].x + bb.x);
    top_insert<P>(top, x[t].y + bb.y);
    top_insert<P>(top, x[t].z + bb.z);
    top_insert<P>(top, x[t].w + bb.w);
  }
  float a;
  if constexpr (S::LPR == 1) {
    a = top[P - 1];
  } else if constexpr (S::LPR == 2) {
    a = top_merge_last<P, kQuadXor1>(top);
  } else {
    top_merge<P, kQuadXor1>(top);
    a = top_merge_last<P, kQuadXor2>(top);
  }
  // alpha is read again only by the next pass: a non-temporal store keeps
  // it from sitting dirty in L2 until the end of the kernel
  if (valid && ql == 0) __builtin_nontemporal_store(a, alpha + row);
  if constexpr (HM == 2) {
    // full 16-bit key histogram, [E][65536] int32 in global memory
    if (valid) {
#pragma unroll
      for (int t = 0; t < S::F4; ++t) {
        const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
        const uint32_t k01 = key2(bf16x2_rne(a - x[t].x, a - x[t].y));
        const uint32_t k23 = key2(bf16x2_rne(a - x[t].z, a - x[t].w));
        int32_t* h = ghist + int64_t(4 * quad) * 65536;
        atomicAdd(h + (k01 & 0xFFFFu), 1);
        atomicAdd(h + 65536 + (k01 >> 16), 1);
        atomicAdd(h + 2 * 65536 + (k23 & 0xFFFFu), 1);
        atomicAdd(h + 3 * 65536 + (k23 >> 16), 1);
      }
    }
  }
  if constexpr (HM == 1) {
    if (valid) {
      uint32_t* h = lds_hist + (S::NC > 1 ? p1_copy<S, PAIR>(rho) * S::HDW : 0);
#pragma unroll
      for (int t = 0; t < S::F4; ++t) {
        const int quad = S::LPR * p1_blk<S, PAIR>(t, rot) + ql;
        const uint32_t swz = hist16_swizzle2(quad);
        hist16_add_hi(h, quad, 0, key2(bf16x2_rne(a - x[t].x, a - x[t].y)) ^ swz);
        hist16_add_hi(h, quad, 2, key2(bf16x2_rne(a - x[t].z, a - x[t].w)) ^ swz);
      }
    }
  }
  // The loads last, after the histogram's key arithmetic, with a scheduling
  // fence between: only the raw scores stay live into the count.
  if constexpr (LOAD) {
    __builtin_amdgcn_sched_barrier(0);
    count_loads<E, P>(x, lds_b, rot, ql, a, K, valid, lds_load);
  }
}

// MB (with LOAD): per-microbatch loads as well.  Each workgroup then takes
// one contiguous block of rows and walks it microbatch by microbatch,
// counting the members of the current microbatch in LDS and adding them to
// load_mb and load at each microbatch boundary (one atomic per non-zero
// counter instead of one device atomic per member).
template <int E, int P, int HM, bool LOAD, bool MB, bool ST = false>
__global__ __launch_bounds__((p1_waves<LOAD, P, MB>() * kWave)) void k_margins_topk(
    const float* __restrict__ s, const float* __restrict__ b, int64_t N, int wg_per_layer, int bdiv, int K,
    float* __restrict__ alpha, int32_t* __restrict__ load, int32_t* __restrict__ hist_hi,
    int32_t* __restrict__ load_mb, int64_t n_mb) {
  using S = P1Shape<E>;
  static_assert(!MB || LOAD, "microbatch loads need load counting");
  constexpr int kWaves = p1_waves<LOAD, P, MB>();
  constexpr int kThreads = kWaves * kWave;
  __shared__ uint32_t lds_hist[HM == 1 ? S::HDW * S::NC : 4];
  __shared__ float lds_b[E];
  __shared__ int32_t lds_load[E];

  const int tid = threadIdx.x;
  const int layer = blockIdx.x / wg_per_layer;
  const int g = blockIdx.x - layer * wg_per_layer;
  s += int64_t(layer) * N * E;
  b += int64_t(layer / bdiv) * E;  // bdiv consecutive layers share a bias row
  alpha += int64_t(layer) * N;
  int32_t* ghist = HM == 2 ? hist_hi + int64_t(layer) * E * 65536 : nullptr;
  if (LOAD) load += int64_t(layer) * E;
  if (MB) load_mb += int64_t(layer) * (N / n_mb) * E;

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int rho = lane / S::LPR;
  const int ql = lane % S::LPR;
  constexpr int64_t kTrip = int64_t(kWaves) * S::WROWS;
  constexpr bool kRoll = QB_P1_ROLL != 0 && HM == 1 && !LOAD && !MB;
  // ST (streaming, for layers far larger than the Infinity Cache): the
  // rolling path reads its rows with non-temporal loads, 8 lanes per row so
  // that every load instruction takes whole 128-byte lines of a row (with 4
  // lanes per row, 64-byte halves of a line, non-temporal loads fetch lines
  // twice).
  static_assert(!ST || (kRoll && E >= 32), "the streaming variant is the rolling path's");
  constexpr int kRL = ST ? 8 : 4;
  constexpr bool kStream = ST;
  constexpr bool kPair = QB_P1_PAIR != 0 && HM == 1 && !LOAD;
  using SR = P1Shape<E, kRL>;
  static_assert(SR::WROWS == S::WROWS, "one trip shape for every row split");
  const int rrho = lane / SR::LPR, rql = lane % SR::LPR;
  float4 xr[SR::U][SR::F4];  // the rolling path's score slots
  if constexpr (kRoll && QB_P1_EARLY) {
    // the first trip's loads go out before the table is cleared
    if (g < (N + kTrip - 1) / kTrip) {
      const int64_t base = int64_t(g) * kTrip + int64_t(wave) * SR::WROWS;
#pragma unroll
      for (int u = 0; u < SR::U; ++u) p1_load<E, kRL, kStream, kPair>(s, base + u * SR::RPW, N, rrho, rql, xr[u]);
    }
  }

  if constexpr (HM == 1) hist16_zero<E * S::NC>(lds_hist, tid, kThreads);
  for (int j = tid; j < E; j += kThreads) {
    lds_b[j] = b[j];
    lds_load[j] = 0;
  }
  __syncthreads();

  if constexpr (!MB) {
    // Block-cyclic trips: this workgroup takes trips g, g + G, g + 2G, ...
    // Every wave runs the same number of trips (rows past N are clamped and
    // masked), and the waves meet at a bare barrier once per trip: kept in
    // step, the workgroup reads each block of rows together (193-195 us
    // against 201-202 us for 1M x 256 when the waves drift apart).  The
    // upper half of the waves issues its loads before the barrier and the
    // lower half after it, so the scores of one half are in flight while
    // the other half still ranks and counts its rows (190-191 us; all waves
    // loading on the same side of the barrier leaves HBM idle while they
    // all compute).  The barrier orders nothing: the histogram atomics need
    // no ordering until the flush, which a full barrier precedes.
    const int64_t trips = (N + kTrip - 1) / kTrip;
    const bool early = wave >= kWaves / 2;
    if constexpr (kRoll) {
      // Rolling refill (p1_rows_roll): the next trip's rows stream in while
      // this trip is counted, with no extra registers; the waves still meet
      // once per trip.  EQB step against the half-and-half loads below:
      // 1,048,576 x 256 371-376 against 373-381 us, 262,144 x 256 111 against
      // 116.5 us, 65,536 x 256 54.7 against 56.9 us; one GiB of scores at
      // E = 16 / 32 / 64 620 / 407 / 410 against 653 / 421 / 420 us; the
      // 48-layer step 4.29 against 4.26-4.28 ms.  Without the barrier: 386-390
      // us at 1M.
      auto& x = xr;
      if (!QB_P1_EARLY && g < trips) {
        const int64_t base = int64_t(g) * kTrip + int64_t(wave) * SR::WROWS;
#pragma unroll
        for (int u = 0; u < SR::U; ++u) p1_load<E, kRL, kStream, kPair>(s, base + u * SR::RPW, N, rrho, rql, x[u]);
      }
      for (int64_t T = g; T < trips; T += wg_per_layer) {
        const int64_t base = T * kTrip + int64_t(wave) * SR::WROWS;
        const int64_t nbase = (T + wg_per_layer) * kTrip + int64_t(wave) * SR::WROWS;
        const bool more = T + wg_per_layer < trips;
        if (QB_P1_ROLL == 1) __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int u = 0; u < SR::U; ++u)
          p1_rows_roll<E, P, kRL, kStream, kPair>(x[u], s, base + u * SR::RPW, nbase + u * SR::RPW, more, N,
                                                  rrho, rql, lds_b, lds_hist, alpha);
      }
    } else
    for (int64_t T = g; T < trips; T += wg_per_layer) {
      const int64_t base = T * kTrip + int64_t(wave) * S::WROWS;
      float4 x[S::U][S::F4];
      if (early) {
#pragma unroll
        for (int u = 0; u < S::U; ++u) p1_load<E, 4, false, kPair>(s, base + u * S::RPW, N, rho, ql, x[u]);
        __builtin_amdgcn_s_barrier();
      } else {
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int u = 0; u < S::U; ++u) p1_load<E, 4, false, kPair>(s, base + u * S::RPW, N, rho, ql, x[u]);
      }
#pragma unroll
      for (int u = 0; u < S::U; ++u)
        p1_rows<E, P, HM, LOAD, kPair>(x[u], base + u * S::RPW, N, rho, ql, lane, K, lds_b, lds_hist, lds_load, alpha,
                                ghist);
    }
  } else {
    // Contiguous block of whole trips, split at microbatch boundaries.
    const int64_t trips = (N + kTrip - 1) / kTrip;
    const int64_t chunk = (trips + wg_per_layer - 1) / wg_per_layer * kTrip;
    const int64_t r0 = int64_t(g) * chunk;
    const int64_t r1 = r0 + chunk < N ? r0 + chunk : N;
    for (int64_t seg0 = r0; seg0 < r1;) {
      const int64_t mb = seg0 / n_mb;
      const int64_t seg1 = (mb + 1) * n_mb < r1 ? (mb + 1) * n_mb : r1;
      for (int64_t base = seg0 + int64_t(wave) * S::WROWS; base < seg1; base += kTrip) {
        float4 x[S::U][S::F4];
#pragma unroll
        for (int u = 0; u < S::U; ++u) p1_load<E>(s, base + u * S::RPW, seg1, rho, ql, x[u]);
#pragma unroll
        for (int u = 0; u < S::U; ++u)
          p1_rows<E, P, HM, LOAD>(x[u], base + u * S::RPW, seg1, rho, ql, lane, K, lds_b, lds_hist, lds_load,
                                  alpha, ghist);
      }
      __syncthreads();
      for (int j = tid; j < E; j += kThreads) {
        const int32_t v = lds_load[j];
        if (v) {
          atomicAdd(load_mb + mb * E + j, v);
          atomicAdd(load + j, v);
          lds_load[j] = 0;
        }
      }
      __syncthreads();
      seg0 = seg1;
    }
  }
  __syncthreads();
  // The high-byte counts crowd into a few adjacent bins per expert, so a
  // 64-bit atomic per bin pair halves the flush's atomics (190 -> 188 us
  // at 1M x 256).
  if constexpr (HM == 1)
    hist16_flush_pairs<E, S::NC>(lds_hist, hist_hi + int64_t(layer) * E * 256, tid, kThreads, g);
  if constexpr (LOAD && !MB) {
    for (int j = tid; j < E; j += kThreads)
      if (lds_load[j]) atomicAdd(load + j, lds_load[j]);
  }
}

template <int E, int P, int HM, bool LOAD, bool MB = false, bool ST = false>
static int launch_p1_v(const float* s, const float* b, int L, int bdiv, int64_t N, int K, float* alpha,
                       int32_t* load, int32_t* hist_hi, hipStream_t st, int32_t* load_mb = nullptr,
                       int64_t n_mb = 1) {
  constexpr int kThreads = p1_waves<LOAD, P, MB>() * kWave;
  const RowSplit sp = split_rows(L, N, p1_waves<LOAD, P, MB>() * P1Shape<E>::WROWS, QB_P1_MAXROWS);
  hipLaunchKernelGGL((k_margins_topk<E, P, HM, LOAD, MB, ST>), dim3(unsigned(sp.blocks)), dim3(kThreads),
                     0, st, s, b, N, sp.wg_per_layer, bdiv, K, alpha, load, hist_hi, load_mb, n_mb);
  return int(hipGetLastError());
}

template <int E, int P>
static int launch_p1(const float* s, const float* b, int L, int bdiv, int64_t N, int K, float* alpha,
                     int32_t* load, int32_t* hist_hi, hipStream_t st, int32_t* load_mb, int64_t n_mb) {
  if (load && load_mb) {
    if (hist_hi)
      return launch_p1_v<E, P, 1, true, true>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
    return launch_p1_v<E, P, 0, true, true>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
  }
  if (hist_hi && load) return launch_p1_v<E, P, 1, true>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st);
  if (hist_hi) {
    // Streaming pays at E = 256 only: with fewer experts the 8 lanes of a
    // row hold 4-16 scores each and the extra merge per row costs more than
    // the faster stream gives (one GiB of scores in pass 1, plain against
    // streaming: E = 32 206 against 268 us, E = 64 211 against 243, E = 128
    // 205 against 214; E = 256 193 against 189).
    if constexpr (E == 256 && QB_P1_ROLL != 0) {
      if (stream_pass(L, N, E))
        return launch_p1_v<E, P, 1, false, false, true>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st);
    }
    return launch_p1_v<E, P, 1, false>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st);
  }
  if (load) return launch_p1_v<E, P, 0, true>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st);
  return launch_p1_v<E, P, 0, false>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st);
}

// List length P = K + 1, 2 .. kMaxList (K <= 15), dispatched at run time.
constexpr int kMaxList = 16;

template <int E, int P = 2>
static int launch_p1_k(const float* s, const float* b, int L, int bdiv, int64_t N, int K, float* alpha,
                       int32_t* load, int32_t* hist_hi, hipStream_t st, int32_t* load_mb, int64_t n_mb) {
  if constexpr (P <= kMaxList) {
    if (K + 1 == P) return launch_p1<E, P>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
    return launch_p1_k<E, P + 1>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
  }
  return int(hipErrorInvalidValue);
}

template <int E, int P = 2>
static int launch_full_k(const float* s, const float* b, int L, int64_t N, int K, float* alpha,
                         int32_t* hist_full, hipStream_t st) {
  if constexpr (P <= kMaxList) {
    if (K + 1 == P) return launch_p1_v<E, P, 2, false>(s, b, L, 1, N, K, alpha, nullptr, hist_full, st);
    return launch_full_k<E, P + 1>(s, b, L, N, K, alpha, hist_full, st);
  }
  return int(hipErrorInvalidValue);
}

#ifndef QB_P1_E
#error "compile with -DQB_P1_E=<experts>: one translation unit per expert count"
#endif

#define QB_P1_CAT2(a, b) a##b
#define QB_P1_CAT(a, b) QB_P1_CAT2(a, b)
int QB_P1_CAT(launch_margins_topk_e, QB_P1_E)(const float* s, const float* b, int L, int bdiv,
                                               int64_t N, int K, float* alpha, int32_t* load,
                                               int32_t* hist_hi, hipStream_t st, int32_t* load_mb,
                                               int64_t n_mb) {
  return launch_p1_k<QB_P1_E>(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
}

int QB_P1_CAT(launch_margins_full_e, QB_P1_E)(const float* s, const float* b, int L, int64_t N, int K,
                                              float* alpha, int32_t* hist_full, hipStream_t st) {
  return launch_full_k<QB_P1_E>(s, b, L, N, K, alpha, hist_full, st);
}

}  // namespace qbk
