// qb_internal.hpp -- launch plumbing shared by the libqb translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbk {

// Work split of a row-chunked pass: blocks = L * wg_per_layer, each block
// owns rows [g * rows_per_wg, min(N, (g+1) * rows_per_wg)) of one layer.
struct RowSplit {
  int rows_per_wg;
  int wg_per_layer;
  int64_t blocks;
};

// step = rows one workgroup consumes per loop trip (its rows_per_wg is a
// multiple of it); cap bounds the packed 16-bit LDS counters (< 65536 tokens
// per workgroup flush) and keeps layers load-balanced.
RowSplit split_rows(int L, int64_t N, int step, int cap);
// N rows of one layer in about `chunks` pieces (multiples of `step`);
// blocks counts one layer.
RowSplit split_rows_chunks(int64_t N, int64_t chunks, int step);

int device_cu_count();

// Launchers (return hipError_t as int).  Shapes were validated by the caller.
int launch_margins_topk(const float* s, const float* b, int L, int64_t N, int E, int K,
                        float* alpha, int32_t* load, int32_t* hist_hi, hipStream_t st);
int launch_radix_hist(bool lo, const float* s, const float* alpha, int L, int64_t N, int E,
                      const int32_t* sel_hi, int32_t* hist, hipStream_t st);
int launch_margin_keys(const float* s, const float* alpha, int L, int64_t N, int E, uint16_t* keys,
                       hipStream_t st);
int launch_select(int phase, int L, int E, int K, const int32_t* hist, int n_bins,
                  int32_t* sel_hi, int32_t* rank_lo, uint16_t* key_out, float* q_out, float* b,
                  float* bounds, int32_t* err, hipStream_t st);
int launch_uniform_hist(const float* s, const float* alpha, int L, int64_t N, int E,
                        const float* bounds, int n_bins, int32_t* hist_u, hipStream_t st);
int launch_bias_bounds(const float* b, int L, int E, float* bounds, hipStream_t st);
int launch_fill_i32(int32_t* dst, int64_t count, int32_t value, hipStream_t st);
int launch_lei(float* g, const int32_t* load, int64_t N, int E, int K, float eta,
               hipStream_t st);

bool supported_E(int E);

}  // namespace qbk
