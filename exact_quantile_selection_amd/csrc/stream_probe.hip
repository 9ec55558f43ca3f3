// stream_probe.hip -- a plain streaming read that bounds the library's passes
// from above: every byte of a buffer is loaded once and a trivial integer
// fold of it is kept live.  It does no work of the method; its achieved GB/s
// is the practical HBM ceiling the quantile-balancing passes (which read the
// score matrix and write almost nothing) are measured against, next to the
// vendor peak.  Diagnostic only: the library's hot path never calls it.
//
// Work split: the buffer is cut into trips of kThreads * U 16-byte items;
// trip t goes to workgroup t % grid (block-cyclic, as the library's passes
// walk their rows), and within a trip lane i of the workgroup loads items
// i, i + kThreads, ..., so every load instruction of a wave covers 1 KiB of
// consecutive bytes.  A workgroup issues all U loads of a trip before it
// uses any of them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/stream_probe.h"

namespace {

constexpr int kThreads = 1024;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT = false>
__global__ __launch_bounds__(kThreads) void k_read(const u32x4* __restrict__ p, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t trip_items = int64_t(kThreads) * U;
  const int64_t stride = int64_t(gridDim.x) * trip_items;
  uint32_t acc = 0;
  for (int64_t base = int64_t(blockIdx.x) * trip_items; base < n16; base += stride) {
    u32x4 v[U];
    if (base + trip_items <= n16) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4* a = p + base + int64_t(u) * kThreads + threadIdx.x;
        v[u] = NT ? __builtin_nontemporal_load(a) : *a;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + int64_t(u) * kThreads + threadIdx.x;
        v[u] = i < n16 ? p[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // a store only when the fold hits one fixed value (practically never):
  // the loads stay live without adding write traffic
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// The same walk, storing every item to dst at its own offset: a plain copy,
// the ceiling of the passes that read and write equal amounts (the LEI
// gradient offsets).
template <int U>
__global__ __launch_bounds__(kThreads) void k_copy(const u32x4* __restrict__ p, u32x4* __restrict__ q,
                                                   int64_t n16) {
  const int64_t trip_items = int64_t(kThreads) * U;
  const int64_t stride = int64_t(gridDim.x) * trip_items;
  for (int64_t base = int64_t(blockIdx.x) * trip_items; base < n16; base += stride) {
    if (base + trip_items <= n16) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = p[base + int64_t(u) * kThreads + threadIdx.x];
#pragma unroll
      for (int u = 0; u < U; ++u) q[base + int64_t(u) * kThreads + threadIdx.x] = v[u];
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + int64_t(u) * kThreads + threadIdx.x;
        if (i < n16) q[i] = p[i];
      }
    }
  }
}

bool bad_args(const void* p, int64_t bytes, int grid) {
  return p == nullptr || bytes < 16 || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(p) % 16) != 0 ||
         grid < 1 || grid > (1 << 20);
}

template <int U, bool NT = false>
void launch_read(const u32x4* q, int64_t n16, int grid, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL((k_read<U, NT>), dim3(grid), dim3(kThreads), 0, st, q, n16, sink);
}

template <int U>
void launch_copy(const u32x4* p, u32x4* q, int64_t n16, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_copy<U>, dim3(grid), dim3(kThreads), 0, st, p, q, n16);
}

}  // namespace

extern "C" {

int sp_read(const void* p, int64_t bytes, int grid, int unroll, uint32_t* sink, sp_stream_t stream) {
  if (bad_args(p, bytes, grid) || sink == nullptr) return SP_EINVAL;
  const u32x4* q = static_cast<const u32x4*>(p);
  const int64_t n16 = bytes / 16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (unroll) {
    case 1: launch_read<1>(q, n16, grid, sink, st); break;
    case 2: launch_read<2>(q, n16, grid, sink, st); break;
    case 4: launch_read<4>(q, n16, grid, sink, st); break;
    case 8: launch_read<8>(q, n16, grid, sink, st); break;
    case 16: launch_read<16>(q, n16, grid, sink, st); break;
    default: return SP_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? SP_OK : SP_EHIP;
}

int sp_read_nt(const void* p, int64_t bytes, int grid, int unroll, uint32_t* sink, sp_stream_t stream) {
  if (bad_args(p, bytes, grid) || sink == nullptr) return SP_EINVAL;
  const u32x4* q = static_cast<const u32x4*>(p);
  const int64_t n16 = bytes / 16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (unroll) {
    case 1: launch_read<1, true>(q, n16, grid, sink, st); break;
    case 2: launch_read<2, true>(q, n16, grid, sink, st); break;
    case 4: launch_read<4, true>(q, n16, grid, sink, st); break;
    case 8: launch_read<8, true>(q, n16, grid, sink, st); break;
    case 16: launch_read<16, true>(q, n16, grid, sink, st); break;
    default: return SP_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? SP_OK : SP_EHIP;
}

int sp_copy(const void* src, void* dst, int64_t bytes, int grid, int unroll, sp_stream_t stream) {
  if (bad_args(src, bytes, grid) || bad_args(dst, bytes, grid)) return SP_EINVAL;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + bytes && b < a + bytes) return SP_EINVAL;  // overlapping buffers
  const u32x4* p = static_cast<const u32x4*>(src);
  u32x4* q = static_cast<u32x4*>(dst);
  const int64_t n16 = bytes / 16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (unroll) {
    case 1: launch_copy<1>(p, q, n16, grid, st); break;
    case 2: launch_copy<2>(p, q, n16, grid, st); break;
    case 4: launch_copy<4>(p, q, n16, grid, st); break;
    case 8: launch_copy<8>(p, q, n16, grid, st); break;
    default: return SP_EINVAL;
  }
  return hipGetLastError() == hipSuccess ? SP_OK : SP_EHIP;
}

}  // extern "C"
