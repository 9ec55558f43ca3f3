// qb_device.hpp -- device building blocks shared by the libqb kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbk {

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));
typedef short s2v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Two fp32 -> two bf16 patterns (round to nearest even, subnormals kept) in
// one v_cvt_pk_bf16_f32: low half = a, high half = b.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  f2v x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2v));
}

// Order-preserving 16-bit key of each bf16 half: negative -> ~u,
// non-negative -> u | 0x8000 (so unsigned key order is value order).
__device__ __forceinline__ uint32_t key2(uint32_t p) {
  s2v x = __builtin_bit_cast(s2v, p);
  s2v sm = x >> (s2v){15, 15};  // 0xFFFF where the half is negative
  uint32_t m = (__builtin_bit_cast(uint32_t, sm) & 0x7FFF7FFFu) | 0x80008000u;
  return p ^ m;
}

// Inverse of the key map for one 16-bit key.
__device__ __forceinline__ uint32_t unkey16(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
}

// Cross-lane move inside a row of 4 lanes (DPP quad_perm).
template <int CTRL>
__device__ __forceinline__ float quad_mov(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int quad_mov_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i of each group of 8 reads lane 7 - i

// Insert v into a descending list t[0..P-1] keeping the P largest values:
// t'_0 = max(t_0, v), t'_k = med3(t_{k-1}, t_k, v).  One VALU op per slot.
template <int P>
__device__ __forceinline__ void top_insert(float (&t)[P], float v) {
#pragma unroll
  for (int k = P - 1; k >= 1; --k) t[k] = __builtin_amdgcn_fmed3f(t[k - 1], t[k], v);
  t[0] = fmaxf(t[0], v);
}

// Compare-exchange for a descending network; positions below PAD hold +inf
// and never move, so exchanges that touch them are skipped at compile time.
template <int PAD, int A, int B, int W>
__device__ __forceinline__ void ce_desc(float (&c)[W]) {
  if constexpr (A >= PAD) {
    const float hi = fmaxf(c[A], c[B]);
    const float lo = fminf(c[A], c[B]);
    c[A] = hi;
    c[B] = lo;
  }
}

// One half-cleaner stage of a bitonic merge of width W at distance D:
// compare-exchange (i, i + D) for every i with bit D clear.
template <int PAD, int D, int W, int I = 0>
__device__ __forceinline__ void bitonic_stage(float (&c)[W]) {
  if constexpr (I < W) {
    if constexpr ((I & D) == 0) ce_desc<PAD, I, I + D, W>(c);
    bitonic_stage<PAD, D, W, I + 1>(c);
  }
}

// Bitonic merge of width W (a power of two): stages at distances W/2, ...,
// 1 sort a bitonic sequence into descending order.
template <int PAD, int W, int D = W / 2>
__device__ __forceinline__ void bitonic_merge(float (&c)[W]) {
  if constexpr (D >= 1) {
    bitonic_stage<PAD, D, W>(c);
    bitonic_merge<PAD, W, D / 2>(c);
  }
}

// Merge this lane's descending list with the partner lane's (DPP control
// CTRL) into the descending list of the P largest of their union.
// max(A_k, B_{P-1-k}) is the top-P multiset in bitonic order (decreasing,
// then increasing); a bitonic merge of width 8 or 16 (front-padded with
// +inf) restores the order.
template <int P, int CTRL>
__device__ __forceinline__ void top_merge(float (&t)[P]) {
  static_assert(P >= 1 && P <= 16, "list length");
  constexpr int W = P <= 8 ? 8 : 16;
  constexpr int PAD = W - P;
  float pt[P];
#pragma unroll
  for (int k = 0; k < P; ++k) pt[k] = quad_mov<CTRL>(t[k]);
  float c[W];
#pragma unroll
  for (int k = 0; k < PAD; ++k) c[k] = __builtin_inff();
#pragma unroll
  for (int k = 0; k < P; ++k) c[PAD + k] = fmaxf(t[k], pt[P - 1 - k]);
  bitonic_merge<PAD, W>(c);
#pragma unroll
  for (int k = 0; k < P; ++k) t[k] = c[PAD + k];
}

// P-th largest of the union of this lane's and the partner's lists: the
// minimum of the top-P multiset max(A_k, B_{P-1-k}).
template <int P, int CTRL>
__device__ __forceinline__ float top_merge_last(const float (&t)[P]) {
  float a = __builtin_inff();
#pragma unroll
  for (int k = 0; k < P; ++k) a = fminf(a, fmaxf(t[k], quad_mov<CTRL>(t[P - 1 - k])));
  return a;
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// A non-temporal (streaming) 16-byte load.
__device__ __forceinline__ float4 ld4_nt(const float* p) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}


__device__ __forceinline__ float comp(const float4& v, int c) {
  return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w));
}

}  // namespace qbk

namespace qbk {

// Packed per-workgroup histogram of E experts x 256 bins in LDS: two 16-bit
// counters per dword.  Expert j = 4*quad + c lives in dword row
// (j >> 1) = 2*quad + (c >> 1), half (j & 1) = (c & 1); the bin is XOR-ed
// with (quad & 63) so the 64 lanes of one instruction, which hold distinct
// quads, land in distinct banks even when their bins coincide.
__device__ __forceinline__ uint32_t hist16_swizzle2(int quad) {
  return uint32_t(quad & 63) * 0x01000100u;  // swizzle for both halves of a key pair
}

// Adds one (key pair) of experts 4*quad + {c0, c0+1} (c0 = 0 or 2) into the
// packed LDS histogram by the high byte of each key.  `kp` is the key pair
// already XOR-ed with hist16_swizzle2(quad).
__device__ __forceinline__ void hist16_add_hi(uint32_t* lds, int quad, int c0, uint32_t kp) {
  uint32_t* rowp = lds + quad * 512 + (c0 >> 1) * 256;
  atomicAdd(rowp + ((kp >> 8) & 0xFFu), 1u);
  atomicAdd(rowp + (kp >> 24), 0x10000u);
}

// Adds the packed LDS histogram into the global int32 histogram
// out[E][256] (non-zero counters only, agent-scope atomics).  The
// workgroups of a pass finish together; each starts its walk at a different
// block of nthreads dwords (`start`, e.g. its index) so that concurrent
// flushes hit different global counters instead of queueing on the same
// ones.
template <int E>
__device__ __forceinline__ void hist16_flush(const uint32_t* lds, int32_t* out, int tid, int nthreads,
                                             int start) {
  constexpr int HDW = (E / 2) * 256;
  const int nblk = (HDW + nthreads - 1) / nthreads;
  const int b0 = start % nblk;
  for (int k = 0; k < nblk; ++k) {
    int blk = b0 + k;
    blk = blk >= nblk ? blk - nblk : blk;
    const int d = blk * nthreads + tid;
    if (d >= HDW) continue;
    const uint32_t v = lds[d];
    if (v) {
      const int pair = d >> 8;
      const int quad = pair >> 1;
      const int h = (d & 255) ^ (quad & 63);
      const int j0 = 2 * pair;
      if (v & 0xFFFFu) atomicAdd(out + j0 * 256 + h, int(v & 0xFFFFu));
      if (v >> 16) atomicAdd(out + (j0 + 1) * 256 + h, int(v >> 16));
    }
  }
}

// As hist16_flush, two adjacent bins of an expert per 64-bit atomic (the
// pair of LDS dwords 2 i, 2 i + 1 holds the bins 2 m, 2 m + 1 of the same
// two experts, in either order).  out must be 8-byte aligned.  Each 32-bit
// half takes its own sum: counts stay below 2^31, so the low half never
// carries into the high one.
// NC > 1: the table is NC copies one after the other (counted by different
// lanes), added here; the copies' counts of one counter sum to at most the
// workgroup's rows (<= 65535), so the packed halves add without carries.
template <int E, int NC = 1>
__device__ __forceinline__ void hist16_flush_pairs(const uint32_t* lds, int32_t* out, int tid, int nthreads,
                                                   int start) {
  constexpr int HDW2 = (E / 2) * 128;
  const int nblk = (HDW2 + nthreads - 1) / nthreads;
  const int b0 = start % nblk;
  const uint2* l2 = reinterpret_cast<const uint2*>(lds);
  for (int k = 0; k < nblk; ++k) {
    int blk = b0 + k;
    blk = blk >= nblk ? blk - nblk : blk;
    const int d2 = blk * nthreads + tid;
    if (d2 >= HDW2) continue;
    uint2 v = l2[d2];
#pragma unroll
    for (int c = 1; c < NC; ++c) {
      const uint2 w = l2[c * HDW2 + d2];
      v.x += w.x;
      v.y += w.y;
    }
    if ((v.x | v.y) == 0u) continue;
    const int d = 2 * d2;
    const int pair = d >> 8;
    const int h0 = (d & 255) ^ ((pair >> 1) & 63);  // bin of dword d; dword d + 1 holds h0 ^ 1
    const int hb = h0 & ~1;
    const uint32_t a = (h0 & 1) ? v.y : v.x;  // bin hb
    const uint32_t c = (h0 & 1) ? v.x : v.y;  // bin hb + 1
    const uint64_t lo = uint64_t(a & 0xFFFFu) | (uint64_t(c & 0xFFFFu) << 32);
    const uint64_t hi = uint64_t(a >> 16) | (uint64_t(c >> 16) << 32);
    const int j0 = 2 * pair;
    if (lo) atomicAdd(reinterpret_cast<unsigned long long*>(out + j0 * 256 + hb), (unsigned long long)lo);
    if (hi) atomicAdd(reinterpret_cast<unsigned long long*>(out + (j0 + 1) * 256 + hb), (unsigned long long)hi);
  }
}

template <int E>
__device__ __forceinline__ void hist16_zero(uint32_t* lds, int tid, int nthreads) {
  constexpr int HDW = (E / 2) * 256;
  uint4* h4 = reinterpret_cast<uint4*>(lds);
  for (int d = tid; d < HDW / 4; d += nthreads) h4[d] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace qbk
