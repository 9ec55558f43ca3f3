// qb_api.hip -- the extern "C" boundary of libqb: argument checks, shape
// dispatch and status reporting.  Every entry point validates its arguments
// on the host, launches asynchronously on the caller's stream and never
// synchronises or allocates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/qb.h"
#include <climits>

#include "qb_internal.hpp"

namespace qbk {

int launch_margins_topk_e16(const float*, const float*, int, int, int64_t, int, float*, int32_t*, int32_t*, hipStream_t, int32_t*, int64_t);
int launch_margins_topk_e32(const float*, const float*, int, int, int64_t, int, float*, int32_t*, int32_t*, hipStream_t, int32_t*, int64_t);
int launch_margins_topk_e64(const float*, const float*, int, int, int64_t, int, float*, int32_t*, int32_t*, hipStream_t, int32_t*, int64_t);
int launch_margins_topk_e128(const float*, const float*, int, int, int64_t, int, float*, int32_t*, int32_t*, hipStream_t, int32_t*, int64_t);
int launch_margins_topk_e256(const float*, const float*, int, int, int64_t, int, float*, int32_t*, int32_t*, hipStream_t, int32_t*, int64_t);

int launch_margins_full_e16(const float*, const float*, int, int64_t, int, float*, int32_t*, hipStream_t);
int launch_margins_full_e32(const float*, const float*, int, int64_t, int, float*, int32_t*, hipStream_t);
int launch_margins_full_e64(const float*, const float*, int, int64_t, int, float*, int32_t*, hipStream_t);
int launch_margins_full_e128(const float*, const float*, int, int64_t, int, float*, int32_t*, hipStream_t);
int launch_margins_full_e256(const float*, const float*, int, int64_t, int, float*, int32_t*, hipStream_t);

int launch_margins_topk(const float* s, const float* b, int L, int64_t N, int E, int K,
                        float* alpha, int32_t* load, int32_t* hist_hi, hipStream_t st, int bdiv,
                        int32_t* load_mb, int64_t n_mb) {
  switch (E) {
    case 16: return launch_margins_topk_e16(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
    case 32: return launch_margins_topk_e32(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
    case 64: return launch_margins_topk_e64(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
    case 128: return launch_margins_topk_e128(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
    case 256: return launch_margins_topk_e256(s, b, L, bdiv, N, K, alpha, load, hist_hi, st, load_mb, n_mb);
  }
  return int(hipErrorInvalidValue);
}

bool supported_E(int E) { return E == 16 || E == 32 || E == 64 || E == 128 || E == 256; }

// Compute units of the current device, cached per device (threads may race
// to fill an entry; they store the same value).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t r = a % b;
    a = b;
    b = r;
  }
  return a;
}

RowSplit split_rows(int L, int64_t N, int step, int64_t max_rows) {
  const int64_t cus = device_cu_count();
  RowSplit r;
  r.trips = (N + step - 1) / step;
  int64_t G = cus / gcd64(int64_t(L), cus);  // L * G = lcm(L, CUs)
  const int64_t max_trips = std::max<int64_t>(1, max_rows / step);
  G = std::max(G, (r.trips + max_trips - 1) / max_trips);
  G = std::min(G, r.trips);
  r.wg_per_layer = int(std::max<int64_t>(1, G));
  r.blocks = int64_t(L) * r.wg_per_layer;
  return r;
}

}  // namespace qbk

namespace {

// Largest K of the top-(K+1) passes (lists of up to 16 per lane).
constexpr int kMaxK = 15;

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return QB_OK;
}

int hip_status(int rc, const char* what) {
  if (rc != int(hipSuccess))
    return fail(QB_EHIP, "%s: HIP launch failed: %s", what, hipGetErrorString(hipError_t(rc)));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Every non-null pointer of the list is a multiple of `a` bytes (a power of
// two): the element alignment of the float, int32 and uint16 arrays.
bool aligned_all(uintptr_t a, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0) return false;
  return true;
}

// The element alignment of a call's 4-byte arrays and 2-byte keys.
int check_elem_align(const char* fn, std::initializer_list<const void*> words, const void* key = nullptr) {
  if (!aligned_all(4, words)) return fail(QB_EINVAL, "%s: float and int32 arrays must be 4-byte aligned", fn);
  if (!aligned_all(2, {key})) return fail(QB_EINVAL, "%s: key_out must be 2-byte aligned", fn);
  return QB_OK;
}

// Common shape checks of the passes over s [L][N][E].
int check_pass(const char* fn, const float* s, int L, int64_t N, int E) {
  if (!s) return fail(QB_EINVAL, "%s: s is NULL (expected float [L][N][E] device pointer)", fn);
  if (!aligned16(s)) return fail(QB_EINVAL, "%s: s must be 16-byte aligned", fn);
  if (L < 1) return fail(QB_EINVAL, "%s: L=%d, expected L >= 1", fn, L);
  if (N < 1 || N > INT32_MAX)
    return fail(QB_EINVAL, "%s: N=%lld, expected 1 <= N < 2^31", fn, (long long)N);
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {16, 32, 64, 128, 256}", fn, E);
  return QB_OK;
}

}  // namespace

extern "C" {

QB_API int qb_margins_topk(const float* s, const float* b, int L, int64_t N, int E, int K,
                           float* alpha, int32_t* load, int32_t* hist_hi, qb_stream_t stream) {
  const char* fn = "qb_margins_topk";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!b) return fail(QB_EINVAL, "%s: b is NULL (expected float [L=%d][E=%d])", fn, L, E);
  if (!alpha) return fail(QB_EINVAL, "%s: alpha is NULL (expected float [L=%d][N=%lld])", fn, L, (long long)N);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (K > kMaxK) return fail(QB_EUNSUPPORTED, "%s: K=%d, compiled for K <= %d", fn, K, kMaxK);
  if (!aligned4(b) || !aligned4(alpha) || (load && !aligned4(load)))
    return fail(QB_EINVAL, "%s: b, alpha and load must be 4-byte aligned", fn);
  if (hist_hi && !aligned8(hist_hi)) return fail(QB_EINVAL, "%s: hist_hi must be 8-byte aligned", fn);
  return hip_status(qbk::launch_margins_topk(s, b, L, N, E, K, alpha, load, hist_hi, stream), fn);
}

QB_API int qb_margins_topk_mb(const float* s, const float* b, int L, int64_t N, int E, int K, float* alpha,
                              int32_t* load, int32_t* hist_hi, int64_t n_mb, int32_t* load_mb,
                              qb_stream_t stream) {
  const char* fn = "qb_margins_topk_mb";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!b || !alpha || !load || !load_mb)
    return fail(QB_EINVAL, "%s: b (float [L=%d][E=%d]), alpha (float [L][N]), load (int32 [L][E]) and load_mb (int32 [L][N/n_mb][E]) are required",
                fn, L, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (K > kMaxK) return fail(QB_EUNSUPPORTED, "%s: K=%d, compiled for K <= %d", fn, K, kMaxK);
  if (n_mb < 1 || N % n_mb != 0)
    return fail(QB_EINVAL, "%s: n_mb=%lld must be >= 1 and divide N=%lld", fn, (long long)n_mb, (long long)N);
  if (!aligned4(b) || !aligned4(alpha) || !aligned4(load) || !aligned4(load_mb))
    return fail(QB_EINVAL, "%s: b, alpha, load and load_mb must be 4-byte aligned", fn);
  if (hist_hi && !aligned8(hist_hi)) return fail(QB_EINVAL, "%s: hist_hi must be 8-byte aligned", fn);
  return hip_status(qbk::launch_margins_topk(s, b, L, N, E, K, alpha, load, hist_hi, stream, 1, load_mb, n_mb),
                    fn);
}

QB_API int qb_microbatch_loads(const float* s, const float* b, int L, int64_t N, int E, int K,
                               int64_t n_mb, float* alpha, int32_t* load_mb, qb_stream_t stream) {
  const char* fn = "qb_microbatch_loads";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!b) return fail(QB_EINVAL, "%s: b is NULL (expected float [L=%d][E=%d])", fn, L, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (K > kMaxK) return fail(QB_EUNSUPPORTED, "%s: K=%d, compiled for K <= %d", fn, K, kMaxK);
  if (n_mb < 1 || N % n_mb != 0)
    return fail(QB_EINVAL, "%s: n_mb=%lld must be >= 1 and divide N=%lld", fn, (long long)n_mb,
                (long long)N);
  const int64_t C = N / n_mb;
  if (int64_t(L) * C > int64_t(INT_MAX))
    return fail(QB_EINVAL, "%s: L * (N / n_mb) = %lld microbatches is too many", fn,
                (long long)(int64_t(L) * C));
  if (!alpha || !load_mb)
    return fail(QB_EINVAL, "%s: alpha (float [L=%d][N=%lld]) and load_mb (int32 [L=%d][C=%lld][E=%d]) are required",
                fn, L, (long long)N, L, (long long)C, E);
  if (!aligned4(b) || !aligned4(alpha) || !aligned4(load_mb))
    return fail(QB_EINVAL, "%s: b, alpha and load_mb must be 4-byte aligned", fn);
  return hip_status(qbk::launch_margins_topk(s, b, int(L * C), n_mb, E, K, alpha, load_mb, nullptr, stream,
                                             int(C)),
                    fn);
}

QB_API int qb_maxvio(const int32_t* load, int L, int C, int E, int K, int64_t n_tok, float* maxvio,
                     float* summary, float* worst, qb_stream_t stream) {
  const char* fn = "qb_maxvio";
  if (L < 1 || C < 1 || E < 1 || K < 1 || K > E || n_tok < 1)
    return fail(QB_EINVAL, "%s: L=%d, C=%d, E=%d, K=%d, n_tok=%lld; expected all >= 1 and K <= E", fn, L, C,
                E, K, (long long)n_tok);
  if (int64_t(L) * C > int64_t(INT_MAX))
    return fail(QB_EINVAL, "%s: L * C = %lld rows is too many", fn, (long long)(int64_t(L) * C));
  if (!load || !maxvio)
    return fail(QB_EINVAL, "%s: load (int32 [L=%d][C=%d][E=%d]) and maxvio (float [L][C]) are required", fn, L,
                C, E);
  if (!aligned4(load) || !aligned4(maxvio) || (summary && !aligned4(summary)) || (worst && !aligned4(worst)))
    return fail(QB_EINVAL, "%s: load, maxvio, summary and worst must be 4-byte aligned", fn);
  return hip_status(qbk::launch_maxvio(load, L, C, E, K, n_tok, maxvio, summary, worst, stream), fn);
}

QB_API int qb_allreduce_sum_i32(int32_t* buf, int R, int64_t M, qb_stream_t stream) {
  const char* fn = "qb_allreduce_sum_i32";
  if (R < 1 || M < 0) return fail(QB_EINVAL, "%s: R=%d, M=%lld; expected R >= 1, M >= 0", fn, R, (long long)M);
  if (M == 0) return QB_OK;
  if (!buf) return fail(QB_EINVAL, "%s: buf is NULL (expected int32 [R=%d][M=%lld])", fn, R, (long long)M);
  if (!aligned4(buf)) return fail(QB_EINVAL, "%s: buf must be 4-byte aligned", fn);
  return hip_status(qbk::launch_allreduce_sum(buf, R, M, stream), fn);
}

QB_API int qb_rank_average(const float* q, int R, int E, float* b, float* bounds, qb_stream_t stream) {
  const char* fn = "qb_rank_average";
  if (R < 1 || E < 1 || E > 16384)
    return fail(QB_EINVAL, "%s: R=%d, E=%d; expected R >= 1, 1 <= E <= 16384", fn, R, E);
  if (!q || !b)
    return fail(QB_EINVAL, "%s: q (float [R=%d][E=%d]) and b (float [E]) are required", fn, R, E);
  if (!aligned4(q) || !aligned4(b) || (bounds && !aligned4(bounds)))
    return fail(QB_EINVAL, "%s: q, b and bounds must be 4-byte aligned", fn);
  return hip_status(qbk::launch_rank_average(q, R, E, b, bounds, stream), fn);
}

QB_API int qb_margins_full_hist(const float* s, const float* b, int L, int64_t N, int E, int K,
                                float* alpha, int32_t* hist_full, qb_stream_t stream) {
  const char* fn = "qb_margins_full_hist";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!b || !alpha || !hist_full)
    return fail(QB_EINVAL, "%s: b (float [L=%d][E=%d]), alpha (float [L][N]) and hist_full (int32 [L][E][65536]) are required",
                fn, L, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (K > kMaxK) return fail(QB_EUNSUPPORTED, "%s: K=%d, compiled for K <= %d", fn, K, kMaxK);
  if (!aligned4(b) || !aligned4(alpha) || !aligned16(hist_full))
    return fail(QB_EINVAL, "%s: b and alpha must be 4-byte and hist_full 16-byte aligned", fn);
  int rc;
  switch (E) {
    case 16: rc = qbk::launch_margins_full_e16(s, b, L, N, K, alpha, hist_full, stream); break;
    case 32: rc = qbk::launch_margins_full_e32(s, b, L, N, K, alpha, hist_full, stream); break;
    case 64: rc = qbk::launch_margins_full_e64(s, b, L, N, K, alpha, hist_full, stream); break;
    case 128: rc = qbk::launch_margins_full_e128(s, b, L, N, K, alpha, hist_full, stream); break;
    default: rc = qbk::launch_margins_full_e256(s, b, L, N, K, alpha, hist_full, stream); break;
  }
  return hip_status(rc, fn);
}

QB_API int qb_lei_backward(const float* g, const float* s, const int32_t* load_mb, int64_t N, int E, int K,
                           int64_t n_mb, float eta, int bounded, float* g_out, float* dlogits,
                           qb_stream_t stream) {
  const char* fn = "qb_lei_backward";
  if (N < 1) return fail(QB_EINVAL, "%s: N=%lld, expected N >= 1", fn, (long long)N);
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {16, 32, 64, 128, 256}", fn, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (n_mb < 1 || N % n_mb != 0)
    return fail(QB_EINVAL, "%s: n_mb=%lld must be >= 1 and divide N=%lld", fn, (long long)n_mb, (long long)N);
  if (N / n_mb > 65535)
    return fail(QB_EINVAL, "%s: N / n_mb = %lld microbatches, at most 65535", fn, (long long)(N / n_mb));
  if (bounded != 0 && bounded != 1) return fail(QB_EINVAL, "%s: bounded=%d, expected 0 or 1", fn, bounded);
  if (!g || !load_mb)
    return fail(QB_EINVAL, "%s: g (float [N=%lld][E=%d]) and load_mb (int32 [N/n_mb][E]) are required", fn,
                (long long)N, E);
  if (!g_out && !dlogits) return fail(QB_EINVAL, "%s: nothing to write (g_out and dlogits are NULL)", fn);
  if (dlogits && !s) return fail(QB_EINVAL, "%s: dlogits needs the scores s (float [N][E])", fn);
  if (!aligned16(g) || (s && !aligned16(s)) || (g_out && !aligned16(g_out)) || (dlogits && !aligned16(dlogits)))
    return fail(QB_EINVAL, "%s: g, s, g_out and dlogits must be 16-byte aligned", fn);
  if (!aligned4(load_mb)) return fail(QB_EINVAL, "%s: load_mb must be 4-byte aligned", fn);
  return hip_status(qbk::launch_lei_bwd(g, s, load_mb, N, E, K, n_mb, eta, bounded, g_out, dlogits, stream), fn);
}

QB_API int64_t qb_hist_lo_workspace_bytes(int L, int64_t N, int E) {
  if (L < 1 || N < 1 || !qbk::supported_E(E)) return QB_EINVAL;
  return qbk::lo_ws_layout(L, E, qbk::radix_wg_per_layer(L, N, E)).bytes;
}

QB_API int qb_radix_hist_lo_ws(const float* s, const float* alpha, int L, int64_t N, int E, const int32_t* sel_hi,
                               void* ws, int64_t ws_bytes, qb_stream_t stream) {
  const char* fn = "qb_radix_hist_lo_ws";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !sel_hi || !ws)
    return fail(QB_EINVAL, "%s: alpha (float [L][N]), sel_hi (int32 [L=%d][E=%d]) and ws are required", fn, L, E);
  const int64_t need = qb_hist_lo_workspace_bytes(L, N, E);
  if (ws_bytes < need)
    return fail(QB_EINVAL, "%s: ws_bytes=%lld, this shape needs %lld (qb_hist_lo_workspace_bytes)", fn,
                (long long)ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(QB_EINVAL, "%s: ws must be 16-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha, sel_hi})) return rc;
  return hip_status(qbk::launch_radix_hist_lo_ws(s, alpha, L, N, E, sel_hi, static_cast<uint8_t*>(ws), stream), fn);
}

QB_API int qb_radix_hist_lo_ws_loads(const float* s, const float* alpha, int L, int64_t N, int E,
                                     const int32_t* sel_hi, void* ws, int64_t ws_bytes, const float* b, int K,
                                     int32_t* load, int64_t n_mb, int32_t* load_mb, qb_stream_t stream) {
  const char* fn = "qb_radix_hist_lo_ws_loads";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !sel_hi || !ws || !b || !load)
    return fail(QB_EINVAL,
                "%s: alpha (float [L][N]), sel_hi (int32 [L=%d][E=%d]), ws, b (float [L][E]) and load (int32 [L][E]) are required",
                fn, L, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  const int64_t need = qb_hist_lo_workspace_bytes(L, N, E);
  if (ws_bytes < need)
    return fail(QB_EINVAL, "%s: ws_bytes=%lld, this shape needs %lld (qb_hist_lo_workspace_bytes)", fn,
                (long long)ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(QB_EINVAL, "%s: ws must be 16-byte aligned", fn);
  if (!aligned4(b) || !aligned4(load) || (load_mb && !aligned4(load_mb)))
    return fail(QB_EINVAL, "%s: b, load and load_mb must be 4-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha, sel_hi})) return rc;
  if (load_mb) {
    const int trip = qbk::radix_lo_trip_rows(E);
    if (n_mb < 1 || N % n_mb != 0 || n_mb % trip != 0)
      return fail(QB_EINVAL, "%s: n_mb=%lld must divide N=%lld and be a multiple of %d rows at E=%d", fn,
                  (long long)n_mb, (long long)N, trip, E);
  }
  return hip_status(qbk::launch_radix_hist_lo_ws_loads(s, alpha, L, N, E, sel_hi, static_cast<uint8_t*>(ws), b, K,
                                                       load, load_mb ? n_mb : 1, load_mb, stream),
                    fn);
}

QB_API int qb_radix_lo_trip_rows(int E) {
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "qb_radix_lo_trip_rows: E=%d, expected E in {16, 32, 64, 128, 256}", E);
  return qbk::radix_lo_trip_rows(E);
}

QB_API int qb_select_lo_ws(int L, int64_t N, int E, const void* ws, int64_t ws_bytes, const int32_t* sel_hi,
                           const int32_t* rank_lo, int32_t* hist_lo, uint16_t* key_out, float* q_out, float* b,
                           float* bounds, int32_t* hist_hi, int32_t* err, qb_stream_t stream) {
  const char* fn = "qb_select_lo_ws";
  if (L < 1 || N < 1) return fail(QB_EINVAL, "%s: L=%d, N=%lld, expected both >= 1", fn, L, (long long)N);
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {16, 32, 64, 128, 256}", fn, E);
  if (!ws || !sel_hi || !rank_lo || !q_out || !b || !bounds)
    return fail(QB_EINVAL,
                "%s: ws, sel_hi, rank_lo (int32 [L=%d][E=%d]), q_out, b (float [L][E]) and bounds (float [L][2]) are required",
                fn, L, E);
  const int64_t need = qb_hist_lo_workspace_bytes(L, N, E);
  if (ws_bytes < need)
    return fail(QB_EINVAL, "%s: ws_bytes=%lld, this shape needs %lld (qb_hist_lo_workspace_bytes)", fn,
                (long long)ws_bytes, (long long)need);
  if (!aligned16(ws) || (hist_lo && !aligned4(hist_lo)) || (hist_hi && !aligned4(hist_hi)))
    return fail(QB_EINVAL, "%s: ws must be 16-byte aligned, hist_lo and hist_hi 4-byte aligned", fn);
  if (int rc = check_elem_align(fn, {sel_hi, rank_lo, q_out, b, bounds, err}, key_out)) return rc;
  return hip_status(qbk::launch_select_lo_ws(L, E, qbk::radix_wg_per_layer(L, N, E), static_cast<const uint8_t*>(ws),
                                             sel_hi, rank_lo, hist_lo, key_out, q_out, b, bounds, hist_hi, err,
                                             stream),
                    fn);
}

}  // extern "C"

namespace {

// Scratch of qb_radix_lo_select_noalloc: the pass-2 partial histograms
// (the workspace of qb_radix_hist_lo_ws) for one group of layers at a time.
// A device array, so the entry point allocates nothing; every GPU the
// library runs on holds its own copy from the first use until the process
// ends.  In host code `scratch` only names the symbol: its device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[QB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call on that device, with that device current).
int scratch_on_current_device(const char* fn, uint8_t** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return fail(QB_EHIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QB_EUNSUPPORTED, "%s: device %d, the scratch table holds devices 0..%d", fn, dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QB_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
  return QB_OK;
}

// Workspace bytes of a group of Lg layers (the same layout and workgroup
// count the launches use for that group).
int64_t group_ws_bytes(int Lg, int64_t N, int E) {
  return qbk::lo_ws_layout(Lg, E, qbk::radix_wg_per_layer(Lg, N, E)).bytes;
}

}  // namespace

extern "C" {

QB_API int qb_radix_lo_select_noalloc(const float* s, const float* alpha, int L, int64_t N, int E,
                                      const int32_t* sel_hi, const int32_t* rank_lo, int32_t* hist_lo,
                                      uint16_t* key_out, float* q_out, float* b, float* bounds, int32_t* hist_hi,
                                      int32_t* err, qb_stream_t stream) {
  const char* fn = "qb_radix_lo_select_noalloc";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !sel_hi || !rank_lo || !q_out || !b || !bounds)
    return fail(QB_EINVAL,
                "%s: alpha (float [L][N]), sel_hi, rank_lo (int32 [L=%d][E=%d]), q_out, b (float [L][E]) and "
                "bounds (float [L][2]) are required",
                fn, L, E);
  if ((hist_lo && !aligned4(hist_lo)) || (hist_hi && !aligned4(hist_hi)))
    return fail(QB_EINVAL, "%s: hist_lo and hist_hi must be 4-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha, sel_hi, rank_lo, q_out, b, bounds, err}, key_out)) return rc;
  const int64_t one = group_ws_bytes(1, N, E);
  if (one > int64_t(QB_NOALLOC_SCRATCH_BYTES))
    return fail(QB_EINVAL,
                "%s: one layer of N=%lld x E=%d needs %lld bytes of scratch, more than the %lld this entry point "
                "holds; use qb_radix_hist_lo_ws with a caller workspace",
                fn, (long long)N, E, (long long)one, (long long)QB_NOALLOC_SCRATCH_BYTES);
  uint8_t* ws = nullptr;
  if (int rc = scratch_on_current_device(fn, &ws)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // Layers in groups whose partials fit the scratch; each group's pass 2 and
  // select run back to back on the stream, so the next group reuses it.
  for (int l0 = 0; l0 < L;) {
    int Lg = L - l0;
    while (Lg > 1 && group_ws_bytes(Lg, N, E) > int64_t(QB_NOALLOC_SCRATCH_BYTES)) --Lg;
    const int G = qbk::radix_wg_per_layer(Lg, N, E);
    const int64_t le = int64_t(l0) * E;
    int rc = qbk::launch_radix_hist_lo_ws(s + int64_t(l0) * N * E, alpha + int64_t(l0) * N, Lg, N, E,
                                          sel_hi + le, ws, st);
    if (rc != int(hipSuccess)) return hip_status(rc, fn);
    rc = qbk::launch_select_lo_ws(Lg, E, G, ws, sel_hi + le, rank_lo + le, hist_lo ? hist_lo + le * 256 : nullptr,
                                  key_out ? key_out + le : nullptr, q_out + le, b + le, bounds + 2 * int64_t(l0),
                                  hist_hi ? hist_hi + le * 256 : nullptr, err, st);
    if (rc != int(hipSuccess)) return hip_status(rc, fn);
    l0 += Lg;
  }
  return ok();
}

QB_API int qb_radix_hist_hi(const float* s, const float* alpha, int L, int64_t N, int E,
                            int32_t* hist_hi, qb_stream_t stream) {
  const char* fn = "qb_radix_hist_hi";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !hist_hi)
    return fail(QB_EINVAL, "%s: alpha (float [L][N]) and hist_hi (int32 [L=%d][E=%d][256]) are required",
                fn, L, E);
  if (!aligned8(hist_hi)) return fail(QB_EINVAL, "%s: hist_hi must be 8-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha})) return rc;
  return hip_status(qbk::launch_radix_hist(false, s, alpha, L, N, E, nullptr, hist_hi, stream), fn);
}

QB_API int qb_radix_hist_lo(const float* s, const float* alpha, int L, int64_t N, int E,
                            const int32_t* sel_hi, int32_t* hist_lo, qb_stream_t stream) {
  const char* fn = "qb_radix_hist_lo";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !sel_hi || !hist_lo)
    return fail(QB_EINVAL,
                "%s: alpha (float [L][N]), sel_hi (int32 [L=%d][E=%d]) and hist_lo (int32 [L][E][256]) are required",
                fn, L, E);
  if (!aligned8(hist_lo)) return fail(QB_EINVAL, "%s: hist_lo must be 8-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha, sel_hi})) return rc;
  return hip_status(qbk::launch_radix_hist(true, s, alpha, L, N, E, sel_hi, hist_lo, stream), fn);
}

QB_API int qb_margin_keys(const float* s, const float* alpha, int L, int64_t N, int E,
                          uint16_t* keys, qb_stream_t stream) {
  const char* fn = "qb_margin_keys";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !keys)
    return fail(QB_EINVAL, "%s: alpha (float [L][N]) and keys (uint16 [L=%d][N][E=%d]) are required", fn,
                L, E);
  if ((reinterpret_cast<uintptr_t>(keys) & 7u) != 0)
    return fail(QB_EINVAL, "%s: keys must be 8-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha})) return rc;
  return hip_status(qbk::launch_margin_keys(s, alpha, L, N, E, keys, stream), fn);
}

QB_API int qb_select_update(int phase, int L, int E, int K, const int32_t* hist, int n_bins,
                            int32_t* sel_hi, int32_t* rank_lo, uint16_t* key_out, float* q_out,
                            float* b, float* bounds, int32_t* err, qb_stream_t stream) {
  const char* fn = "qb_select_update";
  if (L < 1) return fail(QB_EINVAL, "%s: L=%d, expected L >= 1", fn, L);
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {16, 32, 64, 128, 256}", fn, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (!hist) return fail(QB_EINVAL, "%s: hist is NULL", fn);
  switch (phase) {
    case QB_SELECT_HI:
      if (!sel_hi || !rank_lo)
        return fail(QB_EINVAL, "%s(HI): sel_hi and rank_lo (int32 [L=%d][E=%d]) are required", fn, L, E);
      n_bins = 256;
      break;
    case QB_SELECT_LO:
      if (!sel_hi || !rank_lo || !q_out || !b || !bounds)
        return fail(QB_EINVAL,
                    "%s(LO): sel_hi, rank_lo (int32 [L=%d][E=%d]), q_out, b (float [L][E]) and bounds (float [L][2]) are required",
                    fn, L, E);
      n_bins = 256;
      break;
    case QB_SELECT_UNIFORM:
      if (!q_out || !b || !bounds)
        return fail(QB_EINVAL,
                    "%s(UNIFORM): q_out, b (float [L=%d][E=%d]) and bounds (float [L][2]) are required", fn,
                    L, E);
      if (n_bins < 1 || n_bins > 2048)
        return fail(QB_EINVAL, "%s(UNIFORM): n_bins=%d, expected 1 <= n_bins <= 2048", fn, n_bins);
      break;
    case QB_SELECT_FULL:
      if (!q_out || !b || !bounds)
        return fail(QB_EINVAL, "%s(FULL): q_out, b (float [L=%d][E=%d]) and bounds (float [L][2]) are required",
                    fn, L, E);
      if (!aligned16(hist)) return fail(QB_EINVAL, "%s(FULL): hist must be 16-byte aligned", fn);
      n_bins = 65536;
      break;
    default:
      return fail(QB_EINVAL,
                  "%s: phase=%d, expected QB_SELECT_HI, QB_SELECT_LO, QB_SELECT_UNIFORM or QB_SELECT_FULL", fn,
                  phase);
  }
  if (int rc = check_elem_align(fn, {hist, sel_hi, rank_lo, q_out, b, bounds, err}, key_out)) return rc;
  return hip_status(qbk::launch_select(phase, L, E, K, hist, n_bins, sel_hi, rank_lo, key_out, q_out, b,
                                       bounds, err, stream),
                    fn);
}

QB_API int qb_uniform_hist(const float* s, const float* alpha, int L, int64_t N, int E,
                           const float* bounds, int n_bins, int32_t* hist_u, qb_stream_t stream) {
  const char* fn = "qb_uniform_hist";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !bounds || !hist_u)
    return fail(QB_EINVAL,
                "%s: alpha (float [L][N]), bounds (float [L=%d][2]) and hist_u (int32 [L][E=%d][n_bins]) are required",
                fn, L, E);
  if (n_bins < 1 || n_bins > 2048)
    return fail(QB_EINVAL, "%s: n_bins=%d, expected 1 <= n_bins <= 2048", fn, n_bins);
  if (int rc = check_elem_align(fn, {alpha, bounds, hist_u})) return rc;
  return hip_status(qbk::launch_uniform_hist(s, alpha, L, N, E, bounds, n_bins, hist_u, stream), fn);
}

QB_API int64_t qb_uniform_hist_workspace_bytes(int L, int64_t N, int E, int n_bins) {
  if (L < 1 || N < 1 || !qbk::supported_E(E) || n_bins < 1 || n_bins > 2048) return QB_EINVAL;
  return qbk::uh_ws_layout(L, E, qbk::uniform_hist_groups(L, N, E, n_bins), n_bins).bytes;
}

QB_API int qb_uniform_hist_ws(const float* s, const float* alpha, int L, int64_t N, int E, const float* bounds,
                              int n_bins, void* ws, int64_t ws_bytes, qb_stream_t stream) {
  const char* fn = "qb_uniform_hist_ws";
  if (int rc = check_pass(fn, s, L, N, E)) return rc;
  if (!alpha || !bounds || !ws)
    return fail(QB_EINVAL, "%s: alpha (float [L][N]), bounds (float [L=%d][2]) and ws are required", fn, L);
  if (n_bins < 1 || n_bins > 2048)
    return fail(QB_EINVAL, "%s: n_bins=%d, expected 1 <= n_bins <= 2048", fn, n_bins);
  const int64_t need = qb_uniform_hist_workspace_bytes(L, N, E, n_bins);
  if (ws_bytes < need)
    return fail(QB_EINVAL, "%s: ws_bytes=%lld, this shape needs %lld (qb_uniform_hist_workspace_bytes)", fn,
                (long long)ws_bytes, (long long)need);
  if (!aligned16(ws)) return fail(QB_EINVAL, "%s: ws must be 16-byte aligned", fn);
  if (int rc = check_elem_align(fn, {alpha, bounds})) return rc;
  return hip_status(qbk::launch_uniform_hist_ws(s, alpha, L, N, E, bounds, n_bins, static_cast<uint8_t*>(ws), stream),
                    fn);
}

QB_API int qb_select_uniform_ws(int L, int64_t N, int E, int K, int n_bins, const void* ws, int64_t ws_bytes,
                                int32_t* hist_u, float* q_out, float* b, float* bounds, int32_t* err,
                                qb_stream_t stream) {
  const char* fn = "qb_select_uniform_ws";
  if (L < 1 || N < 1) return fail(QB_EINVAL, "%s: L=%d, N=%lld, expected both >= 1", fn, L, (long long)N);
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {16, 32, 64, 128, 256}", fn, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (n_bins < 1 || n_bins > 2048)
    return fail(QB_EINVAL, "%s: n_bins=%d, expected 1 <= n_bins <= 2048", fn, n_bins);
  if (!ws || !q_out || !b || !bounds)
    return fail(QB_EINVAL, "%s: ws, q_out, b (float [L=%d][E=%d]) and bounds (float [L][2]) are required", fn, L, E);
  const int64_t need = qb_uniform_hist_workspace_bytes(L, N, E, n_bins);
  if (ws_bytes < need)
    return fail(QB_EINVAL, "%s: ws_bytes=%lld, this shape needs %lld (qb_uniform_hist_workspace_bytes)", fn,
                (long long)ws_bytes, (long long)need);
  if (!aligned16(ws) || (hist_u && !aligned4(hist_u)) || (err && !aligned4(err)))
    return fail(QB_EINVAL, "%s: ws must be 16-byte aligned, hist_u and err 4-byte aligned", fn);
  if (int rc = check_elem_align(fn, {q_out, b, bounds})) return rc;
  return hip_status(qbk::launch_select_uniform_ws(L, N, E, K, n_bins, qbk::uniform_hist_groups(L, N, E, n_bins),
                                                  static_cast<const uint8_t*>(ws), hist_u, q_out, b, bounds, err,
                                                  stream),
                    fn);
}

QB_API int qb_bias_bounds(const float* b, int L, int E, float* bounds, qb_stream_t stream) {
  const char* fn = "qb_bias_bounds";
  if (!b || !bounds) return fail(QB_EINVAL, "%s: b (float [L][E]) and bounds (float [L][2]) are required", fn);
  if (L < 1 || E < 1) return fail(QB_EINVAL, "%s: L=%d E=%d, expected >= 1", fn, L, E);
  if (int rc = check_elem_align(fn, {b, bounds})) return rc;
  return hip_status(qbk::launch_bias_bounds(b, L, E, bounds, stream), fn);
}

QB_API int qb_fill_i32(int32_t* dst, int64_t count, int32_t value, qb_stream_t stream) {
  const char* fn = "qb_fill_i32";
  if (count < 0) return fail(QB_EINVAL, "%s: count=%lld < 0", fn, (long long)count);
  if (count == 0) return ok();
  if (!dst || !aligned4(dst)) return fail(QB_EINVAL, "%s: dst is NULL or not 4-byte aligned", fn);
  return hip_status(qbk::launch_fill_i32(dst, count, value, stream), fn);
}

QB_API int qb_router_fused(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                           int K, const float* b, float* s_out, float* logits_out, float* alpha,
                           int32_t* load, int32_t* hist_hi, qb_stream_t stream) {
  const char* fn = "qb_router_fused";
  if (!hidden || !w || !b || !s_out || !alpha)
    return fail(QB_EINVAL,
                "%s: hidden (bf16 [N][H]), w (bf16 [E][H]), b (float [E]), s_out (float [N][E]) and alpha "
                "(float [N]) are required",
                fn);
  if (N < 1 || N > INT32_MAX)
    return fail(QB_EINVAL, "%s: N=%lld, expected 1 <= N < 2^31", fn, (long long)N);
  if (H < 64 || H % 64 != 0) return fail(QB_EINVAL, "%s: H=%d, expected a positive multiple of 64", fn, H);
  if (E != 32 && E != 64 && E != 128 && E != 256)
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {32, 64, 128, 256}", fn, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (K > kMaxK) return fail(QB_EUNSUPPORTED, "%s: K=%d, compiled for K <= %d", fn, K, kMaxK);
  if (!aligned16(hidden) || !aligned16(w) || !aligned16(s_out))
    return fail(QB_EINVAL, "%s: hidden, w and s_out must be 16-byte aligned", fn);
  if ((logits_out && !aligned4(logits_out)) || !aligned4(b) || !aligned4(alpha) || (load && !aligned4(load)))
    return fail(QB_EINVAL, "%s: logits_out, b, alpha and load must be 4-byte aligned", fn);
  if (hist_hi && !aligned8(hist_hi)) return fail(QB_EINVAL, "%s: hist_hi must be 8-byte aligned", fn);
  return hip_status(
      qbk::launch_router_fused(hidden, w, N, H, E, s_out, logits_out, b, K, alpha, load, hist_hi, stream), fn);
}

QB_API int qb_router_scores(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E, float* s_out,
                            float* logits_out, qb_stream_t stream) {
  const char* fn = "qb_router_scores";
  if (!hidden || !w || !s_out)
    return fail(QB_EINVAL, "%s: hidden (bf16 [N][H]), w (bf16 [E][H]) and s_out (float [N][E]) are required", fn);
  if (N < 1 || N > INT32_MAX)
    return fail(QB_EINVAL, "%s: N=%lld, expected 1 <= N < 2^31", fn, (long long)N);
  if (H < 64 || H % 64 != 0) return fail(QB_EINVAL, "%s: H=%d, expected a positive multiple of 64", fn, H);
  if (E != 32 && E != 64 && E != 128 && E != 256)
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {32, 64, 128, 256}", fn, E);
  if (!aligned16(hidden) || !aligned16(w) || !aligned16(s_out))
    return fail(QB_EINVAL, "%s: hidden, w and s_out must be 16-byte aligned", fn);
  if (logits_out && !aligned4(logits_out)) return fail(QB_EINVAL, "%s: logits_out must be 4-byte aligned", fn);
  return hip_status(qbk::launch_router_gemm(hidden, w, N, H, E, s_out, logits_out, stream), fn);
}

QB_API int qb_lei_grad(float* g, const int32_t* load, int64_t N, int E, int K, float eta,
                       qb_stream_t stream) {
  const char* fn = "qb_lei_grad";
  if (!g || !load) return fail(QB_EINVAL, "%s: g (float [N][E]) and load (int32 [E]) are required", fn);
  if (!aligned16(g)) return fail(QB_EINVAL, "%s: g must be 16-byte aligned", fn);
  if (N < 1 || N > INT32_MAX)
    return fail(QB_EINVAL, "%s: N=%lld, expected 1 <= N < 2^31", fn, (long long)N);
  if (!qbk::supported_E(E))
    return fail(QB_EUNSUPPORTED, "%s: E=%d, expected E in {16, 32, 64, 128, 256}", fn, E);
  if (K < 1 || K >= E) return fail(QB_EINVAL, "%s: K=%d, expected 1 <= K < E=%d", fn, K, E);
  if (int rc = check_elem_align(fn, {load})) return rc;
  return hip_status(qbk::launch_lei(g, load, N, E, K, eta, stream), fn);
}

QB_API const char* qb_status_string(int status) {
  switch (status) {
    case QB_OK: return "QB_OK";
    case QB_EINVAL: return "QB_EINVAL: invalid argument";
    case QB_EUNSUPPORTED: return "QB_EUNSUPPORTED: shape outside the compiled instantiations";
    case QB_EHIP: return "QB_EHIP: HIP runtime error";
  }
  return "unknown status";
}

QB_API const char* qb_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
