// qb_internal.hpp -- launch plumbing shared by the libqb translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbk {

// Block-cyclic work split of a pass over rows.  A workgroup "trip" is
// `step` consecutive rows; trip t of a layer goes to workgroup t % G, so the
// workgroups in flight at any moment read neighbouring blocks (all HBM
// channels busy) instead of each streaming its own distant chunk.  G is
// chosen so that L * G is a multiple of the CU count where possible, and
// large enough that no workgroup sees more than `max_rows` rows (the packed
// 16-bit LDS counters hold < 65536 per flush).
struct RowSplit {
  int64_t trips;     // trips per layer = ceil(N / step)
  int wg_per_layer;  // G
  int64_t blocks;    // L * G
};
RowSplit split_rows(int L, int64_t N, int step, int64_t max_rows);

int device_cu_count();

// A pass over this many bytes of scores per launch (at least three times the
// MI355X's 256 MiB Infinity Cache) reads them with non-temporal loads: the
// cache cannot hand much of such a layer from one pass to the next, and the
// non-temporal stream is faster (the stream probe reads 1 GiB at 7.0 TB/s
// with them against 6.3 without).  Smaller layers keep the cached loads, so
// that the next pass finds the rows the last one read.
#ifndef QB_STREAM_BYTES
#define QB_STREAM_BYTES (768LL << 20)
#endif
inline bool stream_pass(int L, int64_t N, int E) { return int64_t(L) * N * E * 4 >= QB_STREAM_BYTES; }

// Launchers (return hipError_t as int).  Shapes were validated by the caller.
// bdiv: that many consecutive layers share one bias row (1: one row per
// layer; C: layers are the C microbatches of one layer).
// load_mb (nullable, needs load): also count each token's top-K experts
// into load_mb[l][row / n_mb][e] with device atomics.
int launch_margins_topk(const float* s, const float* b, int L, int64_t N, int E, int K,
                        float* alpha, int32_t* load, int32_t* hist_hi, hipStream_t st, int bdiv = 1,
                        int32_t* load_mb = nullptr, int64_t n_mb = 1);
int radix_wg_per_layer(int L, int64_t N, int E);

// Workspace of the low-byte pass: one partial histogram row per (layer,
// expert, workgroup), row r = (layer * E + j) * G + g.  A row whose 256
// counts are all <= 255 is stored as bytes (p8: uint8 [rows][256]); any
// other as uint16 (p16: uint16 [rows][256]); flag[r] (uint8) says which.
// Every row's flag is written on every pass, so the contents on entry do
// not matter.
struct LoWs {
  int64_t flag;   // byte offset of the flags
  int64_t p16;    // byte offset of the uint16 rows (16-byte aligned)
  int64_t bytes;  // total
};
inline LoWs lo_ws_layout(int L, int E, int G) {
  const int64_t rows = int64_t(L) * E * G;
  LoWs w;
  w.flag = rows * 256;
  w.p16 = (w.flag + rows + 15) / 16 * 16;
  w.bytes = w.p16 + rows * 512;
  return w;
}
int launch_radix_hist_lo_ws(const float* s, const float* alpha, int L, int64_t N, int E,
                            const int32_t* sel_hi, uint8_t* ws, hipStream_t st);
int launch_radix_hist_lo_ws_loads(const float* s, const float* alpha, int L, int64_t N, int E,
                                  const int32_t* sel_hi, uint8_t* ws, const float* b, int K, int32_t* load,
                                  int64_t n_mb, int32_t* load_mb, hipStream_t st);
int radix_lo_trip_rows(int E);
int launch_select_lo_ws(int L, int E, int G, const uint8_t* ws, const int32_t* sel_hi, const int32_t* rank_lo,
                        int32_t* hist_lo, uint16_t* key_out, float* q_out, float* b, float* bounds,
                        int32_t* hist_hi, int32_t* err, hipStream_t st);
int launch_lei_bwd(const float* g, const float* s, const int32_t* load_mb, int64_t N, int E, int K,
                   int64_t n_mb, float eta, int bounded, float* g_out, float* dlogits, hipStream_t st);
int launch_allreduce_sum(int32_t* buf, int R, int64_t M, hipStream_t st);
int launch_rank_average(const float* q, int R, int E, float* b, float* bounds, hipStream_t st);
int launch_maxvio(const int32_t* load, int L, int C, int E, int K, int64_t n_tok, float* v,
                  float* summary, float* worst, hipStream_t st);
int launch_radix_hist(bool lo, const float* s, const float* alpha, int L, int64_t N, int E,
                      const int32_t* sel_hi, int32_t* hist, hipStream_t st);
int launch_margin_keys(const float* s, const float* alpha, int L, int64_t N, int E, uint16_t* keys,
                       hipStream_t st);
int launch_select(int phase, int L, int E, int K, const int32_t* hist, int n_bins,
                  int32_t* sel_hi, int32_t* rank_lo, uint16_t* key_out, float* q_out, float* b,
                  float* bounds, int32_t* err, hipStream_t st);
// Workspace of the K3 binning pass: one partial row of n_bins counts per
// (layer, expert j, workgroup g of j's slice), row r = (layer * E + j) * G +
// g, G = uniform_hist_groups(...).  A row whose counts are all <= 255 is
// stored as bytes (p8: rows of b8 bytes), any other as uint16 (p16: rows of
// b16 bytes); flag[r] says which.  Every row's flag is written on every
// pass, so the contents on entry do not matter.
struct UhWs {
  int64_t rows, b8, b16;  // row count, byte stride of the byte / uint16 rows
  int64_t flag, p8, p16;  // byte offsets (256-aligned)
  int64_t bytes;          // total
};
inline UhWs uh_ws_layout(int L, int E, int64_t G, int n_bins) {
  UhWs w;
  w.rows = int64_t(L) * E * G;
  w.b8 = (int64_t(n_bins) + 15) / 16 * 16;
  w.b16 = (2 * int64_t(n_bins) + 15) / 16 * 16;
  w.flag = 0;
  w.p8 = (w.rows + 255) / 256 * 256;
  w.p16 = w.p8 + (w.rows * w.b8 + 255) / 256 * 256;
  w.bytes = w.p16 + w.rows * w.b16;
  return w;
}
int64_t uniform_hist_groups(int L, int64_t N, int E, int n_bins);
int launch_uniform_hist_ws(const float* s, const float* alpha, int L, int64_t N, int E, const float* bounds,
                           int n_bins, uint8_t* ws, hipStream_t st);
int launch_select_uniform_ws(int L, int64_t N, int E, int K, int n_bins, int64_t G, const uint8_t* ws,
                             int32_t* hist_u, float* q_out, float* b, float* bounds, int32_t* err, hipStream_t st);
int launch_uniform_hist(const float* s, const float* alpha, int L, int64_t N, int E,
                        const float* bounds, int n_bins, int32_t* hist_u, hipStream_t st);
int launch_bias_bounds(const float* b, int L, int E, float* bounds, hipStream_t st);
int launch_fill_i32(int32_t* dst, int64_t count, int32_t value, hipStream_t st);
int launch_router_gemm(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                       float* s_out, float* logits_out, hipStream_t st);
int launch_router_fused(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E, float* s_out,
                        float* logits_out, const float* b, int K, float* alpha, int32_t* load, int32_t* hist_hi,
                        hipStream_t st);
int launch_lei(float* g, const int32_t* load, int64_t N, int E, int K, float eta,
               hipStream_t st);

bool supported_E(int E);

}  // namespace qbk
