/*
 * qb.h -- C ABI of libqb, the MI355X (gfx950) quantile-balancing bias update
 * for an auxiliary-loss-free MoE router.
 *
 * What is computed (per layer, N tokens, E experts, top-K routing):
 *   alpha[i]   = (K+1)-th largest of s[i,:] + b[:] (duplicates counted)
 *   r[i,j]     = fl32(alpha[i] - s[i,j])
 *   key[i,j]   = order-preserving 16-bit key of bf16_rne(r[i,j])
 *   q[j]       = value of the key of rank m = ceil(K*N/E) in expert j's column
 *   b_next[j]  = fl32((double)q[j] - mean_j (double)q[j]); written over b
 *   bounds     = [fl32(min b_next - 1), fl32(max b_next + 1)]
 * Sources: "[Dev] Add global-batch quantile balancing" (Megatron-LM pull
 * request #6637), sections "Quantile estimator" and "Implementation"; "Exact
 * Quantile Balancing and Load-Error Injection for Mixture-of-Experts" (paper
 * summary page), EQB paragraph (two-pass byte radix select over the bf16
 * margins) and LEI paragraph.
 *
 * The exact quantile is reached in two passes over the score matrix:
 *   1. qb_margins_topk (alpha + high-byte histogram of the keys)
 *   2. qb_select_update(QB_SELECT_HI)   -> high byte + residual rank per expert
 *   3. qb_radix_hist_lo                 (low-byte histogram inside that bin)
 *   4. qb_select_update(QB_SELECT_LO)   -> key, q, b_next in place, bounds
 * The K3 mode (1000 uniform bins over the current bounds) is
 *   qb_margins_topk (alpha only) -> qb_uniform_hist -> qb_select_update(UNIFORM),
 * or, merged through a workspace, qb_uniform_hist_ws -> qb_select_uniform_ws.
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers owned by the caller; the library keeps no
 *     reference after the call returns and allocates no memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronises the host, so a sequence of calls can be
 *     captured in a HIP graph.
 *   - Arrays are dense row-major with layers outermost:
 *       s       float  [L][N][E]   (16-byte aligned; one token's scores contiguous)
 *       b       float  [L][E]
 *       alpha   float  [L][N]
 *       load    int32  [L][E]
 *       hist_hi int32  [L][E][256], hist_lo int32 [L][E][256]  (8-byte aligned)
 *       hist_u  int32  [L][E][n_bins]
 *       sel_hi, rank_lo int32 [L][E];  key_out uint16 [L][E]; q_out float [L][E]
 *       bounds  float  [L][2]  ({lo, hi})
 *     Every array is aligned at least to its element (4 bytes; 2 for the
 *     uint16 keys); the larger alignments above and in each call's notes
 *     come on top.  A misaligned pointer is QB_EINVAL.
 *   - Histograms and loads are ACCUMULATED (+=) so that several token chunks
 *     (microbatches) of one global batch can be added into one buffer.  The
 *     caller clears them in place (qb_fill_i32) after the update; buffer
 *     addresses never change.  Accumulated counts must stay below 2^31 (the
 *     int32 range): the high-byte and K3 histograms are flushed with 64-bit
 *     atomics over two adjacent bins, exact only while no low half carries.
 *   - Scores are sigmoid outputs: finite, >= +0.  Bias values are finite.
 *     NaN/Inf inputs give unspecified (but memory-safe) results.
 *   - Supported shapes: E in {16, 32, 64, 128, 256}; 1 <= K <= 15 and K < E;
 *     1 <= N < 2^31; L >= 1; n_bins in [1, 2048].
 *   - Return value: QB_OK, or a negative status; on error nothing is launched.
 *     qb_status_string() names a status; qb_last_error() gives the detailed
 *     message of the calling thread's last failed call (expected shapes
 *     included).
 */
#ifndef QB_H
#define QB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QB_API __attribute__((visibility("default")))

typedef struct ihipStream_t* qb_stream_t; /* same type as hipStream_t */

enum {
  QB_OK = 0,
  QB_EINVAL = -1,       /* null required pointer, bad size, bad alignment */
  QB_EUNSUPPORTED = -2, /* E or K outside the compiled instantiations */
  QB_EHIP = -3          /* the HIP runtime refused the launch */
};

enum { QB_SELECT_HI = 0, QB_SELECT_LO = 1, QB_SELECT_UNIFORM = 2, QB_SELECT_FULL = 3 };

/* Device-side error bits OR-ed into qb_select_update's optional err word. */
enum {
  QB_ERR_ROW_TOTALS = 1, /* expert rows of the histogram do not share one total */
  QB_ERR_EMPTY = 2,      /* the histogram holds no token */
  QB_ERR_RANK = 4        /* no bin reaches the rank (histogram inconsistent) */
};

/*
 * Pass 1.  For every token: v_j = fl32(s_ij + b_j); alpha_i = (K+1)-th
 * largest v (IEEE totalOrder, duplicates counted).  "[Dev] Add global-batch
 * quantile balancing", section "Quantile estimator".
 *   alpha   out [L][N], overwritten.
 *   load    nullable; += 1 for each expert among the first K of the order
 *           (larger v first, equal v by lower expert index).  These are the
 *           per-expert top-K counts the LEI paragraph of the EQB summary page
 *           turns into relative load errors.
 *   hist_hi nullable; if given, hist_hi[l][j][key_ij >> 8] += 1 for every
 *           (i, j) -- the first radix pass of the EQB paragraph, fused so the
 *           scores are read once here.
 */
QB_API int qb_margins_topk(const float* s, const float* b, int L, int64_t N, int E, int K,
                           float* alpha, int32_t* load, int32_t* hist_hi, qb_stream_t stream);

/*
 * First radix pass from a precomputed alpha (EQB paragraph):
 * hist_hi[l][j][key_ij >> 8] += 1 with key from r = fl32(alpha_i - s_ij).
 */
QB_API int qb_radix_hist_hi(const float* s, const float* alpha, int L, int64_t N, int E,
                            int32_t* hist_hi, qb_stream_t stream);

/*
 * Second radix pass (EQB paragraph): for keys whose high byte equals
 * sel_hi[l][j] (from QB_SELECT_HI), hist_lo[l][j][key & 0xFF] += 1.
 * sel_hi entries < 0 (invalid selection) match nothing.
 */
QB_API int qb_radix_hist_lo(const float* s, const float* alpha, int L, int64_t N, int E,
                            const int32_t* sel_hi, int32_t* hist_lo, qb_stream_t stream);

/*
 * The 16-bit keys themselves, keys[l][i][j] = key of bf16_rne(fl32(alpha_i -
 * s_ij)) (EQB paragraph: bf16 bit patterns, order-preserving), uint16
 * [L][N][E], 8-byte aligned.  For inspection and for callers that keep the
 * keys instead of re-reading the scores.
 */
QB_API int qb_margin_keys(const float* s, const float* alpha, int L, int64_t N, int E,
                          uint16_t* keys, qb_stream_t stream);

/*
 * One-pass alternative to the two byte histograms, for comparison ("Exact
 * Quantile Balancing and Load-Error Injection for Mixture-of-Experts",
 * summary page, EQB paragraph: a full 65,536-bin histogram per expert would
 * take 128x the memory of the two 256-bin ones).  Computes alpha as
 * qb_margins_topk does and, in the same pass over s, hist_full[l][j][key] +=
 * 1 for every element's 16-bit margin key (one device atomic per element);
 * QB_SELECT_FULL then reads the quantile straight from it.
 *   s float [L][N][E]; b float [L][E]; alpha float [L][N];
 *   hist_full int32 [L][E][65536] (16-byte aligned; 64 MiB per layer at
 *   E = 256), accumulated (+=).
 */
QB_API int qb_margins_full_hist(const float* s, const float* b, int L, int64_t N, int E, int K,
                                float* alpha, int32_t* hist_full, qb_stream_t stream);

/*
 * Rank scans and the bias update, one workgroup per layer.  The token count
 * is read from expert 0's histogram row (every token adds exactly one margin
 * per expert: review thread of Megatron-LM PR #6637); m = ceil(K * total / E).
 *   QB_SELECT_HI:  hist = hist_hi.  sel_hi[l][j] = first bin h whose running
 *                  count reaches m; rank_lo[l][j] = m - count below h.
 *   QB_SELECT_LO:  hist = hist_lo; reads sel_hi, rank_lo.  key = sel_hi << 8 |
 *                  first low byte whose running count reaches rank_lo; q =
 *                  bf16 value of the key; b <- q - mean(q) (float64 mean in
 *                  expert order, rounded once); bounds <- [min - 1, max + 1].
 *                  ("Quantile estimator": b_next and its mean-centring; the
 *                  in-place update of "Implementation".)
 *   QB_SELECT_UNIFORM: hist = hist_u with n_bins bins over the CURRENT bounds
 *                  (read, then overwritten with the next range); q = lo + w *
 *                  (c + (m - below) / count[c]) in float64 (w = (hi-lo)/n_bins,
 *                  c = first bin reaching m), then centring as above.
 *   QB_SELECT_FULL: hist = a full 16-bit key histogram [L][E][65536]
 *                  (qb_margins_full_hist; n_bins is ignored; 16-byte
 *                  aligned); key = first bin whose running count reaches
 *                  m = ceil(K * T / E), T = the row's own total; q, b and
 *                  bounds as in LO.
 *   q_out: required for LO, UNIFORM and FULL (receives q; NaN marks an expert
 *   whose rank search failed).  key_out, err: nullable.  err receives
 *   QB_ERR_* bits (atomic OR); a layer with a failed expert keeps its b and
 *   bounds unchanged.  HI is one launch (one wave per expert row); LO and
 *   UNIFORM add a per-layer launch for the mean and the bounds.
 */
QB_API int qb_select_update(int phase, int L, int E, int K, const int32_t* hist, int n_bins,
                            int32_t* sel_hi, int32_t* rank_lo, uint16_t* key_out,
                            float* q_out, float* b, float* bounds, int32_t* err,
                            qb_stream_t stream);

/*
 * Pass 2 and the low-byte select without global atomics, for one update per
 * call (no accumulation across calls).  Same results as qb_radix_hist_lo +
 * qb_select_update(QB_SELECT_LO), bit for bit: every workgroup of pass 2
 * stores its counts as a dense partial histogram row per expert in a caller
 * workspace (G = workgroups per layer; a row whose 256 counts are all
 * <= 255 as uint8, any other as uint16, with a byte flag per row saying
 * which), and the select sums the G partials of each bin in workgroup
 * order (integer sums) before the rank scan.  The EQB paragraph's low-byte
 * histogram, with the merge moved from global atomics to the select.
 *   qb_hist_lo_workspace_bytes: bytes the workspace needs for this shape
 *     (L * E * G * 769 rounded up to 16; 48 MiB for one 1,048,576 x 256
 *     layer, of which a pass whose rows all fit in bytes writes 16 MiB), or
 *     a negative status.  ws must be 16-byte aligned; its contents on entry
 *     do not matter (every row's flag is written).
 *   qb_radix_hist_lo_ws: as qb_radix_hist_lo, writing ws (overwritten).
 *   qb_select_lo_ws: as qb_select_update(QB_SELECT_LO) from ws (ws_bytes
 *     at least qb_hist_lo_workspace_bytes, so that a wrong N cannot read
 *     past it); ws must be the workspace the preceding qb_radix_hist_lo_ws
 *     call wrote, with the same L, N and E.  hist_lo (nullable) receives
 *     the summed histogram (overwritten, not accumulated).  hist_hi (nullable, int32
 *     [L][E][256]): the high-byte histogram this update was selected from;
 *     it is zeroed in place (addresses unchanged) -- the reset that follows
 *     the bias update in the "Implementation" section -- so the next pass 1
 *     can accumulate into it without a separate clear.
 */
QB_API int64_t qb_hist_lo_workspace_bytes(int L, int64_t N, int E);
QB_API int qb_radix_hist_lo_ws(const float* s, const float* alpha, int L, int64_t N, int E, const int32_t* sel_hi,
                               void* ws, int64_t ws_bytes, qb_stream_t stream);
QB_API int qb_select_lo_ws(int L, int64_t N, int E, const void* ws, int64_t ws_bytes, const int32_t* sel_hi,
                           const int32_t* rank_lo, int32_t* hist_lo, uint16_t* key_out, float* q_out, float* b,
                           float* bounds, int32_t* hist_hi, int32_t* err, qb_stream_t stream);

/*
 * qb_radix_hist_lo_ws that also counts the top-K loads on its read of the
 * scores, so that pass 1 can run without them (the loads the LEI paragraph
 * of the EQB summary page turns into relative load errors; membership as in
 * qb_margins_topk: v = fl32(s_ij + b_j) above alpha_i, then the values equal
 * to alpha_i by lower expert index up to K).
 *   b float [L][E]: the bias pass 1 computed alpha with (read before the
 *   low-byte select updates it), K that pass's K (1 <= K < E).
 *   load int32 [L][E], required, accumulated (+=).
 *   load_mb nullable, int32 [L][N / n_mb][E], accumulated (+=): the loads of
 *   each microbatch of n_mb consecutive tokens, as qb_microbatch_loads.  n_mb
 *   must divide N and be a multiple of the pass's row trip, max(256,
 *   32768 / E) rows (every multiple of 2048 is); ignored when load_mb is
 *   NULL.
 * Results equal qb_margins_topk's and qb_microbatch_loads' for the same s,
 * b, K and alpha, bit for bit.  QB_EINVAL for a NULL b or load, K out of
 * range, an n_mb that breaks the rules above or unaligned (4-byte) b, load
 * or load_mb; the workspace rules of qb_radix_hist_lo_ws apply.
 */
QB_API int qb_radix_hist_lo_ws_loads(const float* s, const float* alpha, int L, int64_t N, int E,
                                     const int32_t* sel_hi, void* ws, int64_t ws_bytes, const float* b, int K,
                                     int32_t* load, int64_t n_mb, int32_t* load_mb, qb_stream_t stream);
/* That row trip at E experts, max(256, 32768 / E), or QB_EUNSUPPORTED. */
QB_API int qb_radix_lo_trip_rows(int E);

/*
 * qb_radix_hist_lo_ws followed by qb_select_lo_ws, with the workspace taken
 * from a device array inside the library instead of the caller: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * and outputs as that pair of calls (hist_lo, key_out, hist_hi and err
 * nullable; hist_hi zeroed in place when given), bit for bit.
 *   The array holds QB_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the
 *   library runs on, from the first call on that GPU until the process
 *   ends.  Layers are processed in groups whose partial histograms fit it
 *   (one 1,048,576 x 256 layer needs 48 MiB; 48 layers of 262,144 x 256
 *   go in two groups, of 32 and 16); a shape where a single layer does not fit
 *   (qb_hist_lo_workspace_bytes(1, N, E) > QB_NOALLOC_SCRATCH_BYTES) is
 *   rejected with QB_EINVAL.  The contents on entry do not matter (every
 *   partial row is written before it is read), so nothing is cleared.
 *   Every call on one GPU shares that GPU's array: calls that overlap on
 *   one GPU (on different streams, or from different threads) race and
 *   give wrong results; order them on one stream.  Nothing is allocated:
 *   no hipMalloc, no hipFree.
 */
#define QB_NOALLOC_SCRATCH_BYTES (64LL << 20)
QB_API int qb_radix_lo_select_noalloc(const float* s, const float* alpha, int L, int64_t N, int E,
                                      const int32_t* sel_hi, const int32_t* rank_lo, int32_t* hist_lo,
                                      uint16_t* key_out, float* q_out, float* b, float* bounds, int32_t* hist_hi,
                                      int32_t* err, qb_stream_t stream);

/*
 * K3 mode binning ("[Dev] Add global-batch quantile balancing", sections
 * "Quantile estimator" and "Implementation"): for the fp32 margin r,
 * bin = clamp(floor(fl32(fl32(r - lo) * fl32(n_bins / fl32(hi - lo)))), 0,
 * n_bins - 1) with {lo, hi} = bounds[l]; hist_u[l][j][bin] += 1.
 */
QB_API int qb_uniform_hist(const float* s, const float* alpha, int L, int64_t N, int E,
                           const float* bounds, int n_bins, int32_t* hist_u, qb_stream_t stream);

/*
 * K3 with the merge moved from global atomics to the select, as the EQB
 * workspace pair does for the low-byte histogram: every workgroup of the
 * binning pass stores its counts as one partial row per expert in a caller
 * workspace (a row whose n_bins counts are all <= 255 as uint8, any other as
 * uint16, with a byte flag per row), and the select sums each expert's
 * partial rows (integer sums) before the rank scan and the in-bin
 * interpolation of qb_select_update(QB_SELECT_UNIFORM), then updates b and
 * bounds in place.  Same q, b and bounds, bit for bit, as qb_uniform_hist
 * into a zeroed hist_u + qb_select_update(QB_SELECT_UNIFORM); nothing needs
 * zeroing.
 *   qb_uniform_hist_workspace_bytes: bytes the workspace needs for this shape
 *     (49 MB at 1,048,576 x 256 x 1000 bins, 25 MB at 65,536 tokens), or a
 *     negative status.
 *   qb_uniform_hist_ws: as qb_uniform_hist, writing ws (16-byte aligned;
 *     overwritten, every row's flag written).
 *   qb_select_uniform_ws: ws from the preceding qb_uniform_hist_ws with the
 *     same L, N, E and n_bins; the rank is ceil(K N / E) (every token adds
 *     one margin per expert), and an expert whose counts do not sum to N
 *     gets QB_ERR_ROW_TOTALS and q = NaN (its layer is then left
 *     unchanged, as in qb_select_update).  hist_u (nullable, int32
 *     [L][E][n_bins]) receives the summed histogram (overwritten).
 *   qb_select_uniform_ws takes the workspace's size (ws_bytes) and refuses
 *   one smaller than the shape needs, so that a wrong N cannot read past it.
 */
QB_API int64_t qb_uniform_hist_workspace_bytes(int L, int64_t N, int E, int n_bins);
QB_API int qb_uniform_hist_ws(const float* s, const float* alpha, int L, int64_t N, int E, const float* bounds,
                              int n_bins, void* ws, int64_t ws_bytes, qb_stream_t stream);
QB_API int qb_select_uniform_ws(int L, int64_t N, int E, int K, int n_bins, const void* ws, int64_t ws_bytes,
                                int32_t* hist_u, float* q_out, float* b, float* bounds, int32_t* err,
                                qb_stream_t stream);

/*
 * Histogram range from a bias vector: bounds[l] = {fl32(min b - 1),
 * fl32(max b + 1)} (section "Quantile estimator").  Seeds the K3 mode.
 */
QB_API int qb_bias_bounds(const float* b, int L, int E, float* bounds, qb_stream_t stream);

/*
 * In-place reset of int32 buffers (histograms, loads) by a fill kernel, so a
 * captured graph holds no memset node.  "Implementation": reset the
 * histogram without changing buffer addresses.
 */
QB_API int qb_fill_i32(int32_t* dst, int64_t count, int32_t value, qb_stream_t stream);

/*
 * Router forward with pass 1 fused into the GEMM's epilogue, for one layer
 * ("[Dev] Add global-batch quantile balancing", section "Implementation":
 * the fused routing path classifies bins and adds histogram atomics in the
 * router kernel itself; its Validation section exercises the router
 * forward).  logits = hidden . w^T on MFMA (bf16 inputs, fp32 accumulation);
 * s = 1 / (1 + 2^(-x log2 e)) with a two-constant (Cody-Waite) split of
 * x log2 e, the hardware exp2 and reciprocal (within a few ulp of the
 * correctly rounded sigmoid; results below 2^-126 flush to 0), written to
 * s_out.  Each workgroup then reads its just-written rows back (from L2)
 * and computes, as qb_margins_topk does on s_out -- same results bit for
 * bit: alpha, the top-K loads (load += ...) and the high-byte histogram of
 * the bf16 margin keys (hist_hi += ...), counted in LDS and flushed with
 * device atomics; no second pass over the scores.
 *   hidden  uint16 bf16 bit patterns [N][H], 16-byte aligned, H % 64 == 0
 *   w       uint16 bf16 bit patterns [E][H] (nn.Linear weight layout)
 *   b       float [E]; s_out float [N][E] (16-byte aligned);
 *   logits_out nullable float [N][E]; alpha float [N]; load nullable int32 [E];
 *   hist_hi nullable int32 [E][256] (8-byte aligned).
 *   E in {32, 64, 128, 256}; 1 <= K <= 15.
 */
QB_API int qb_router_fused(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                           int K, const float* b, float* s_out, float* logits_out, float* alpha,
                           int32_t* load, int32_t* hist_hi, qb_stream_t stream);

/*
 * The router GEMM and sigmoid of qb_router_fused alone (s_out and the
 * optional logits_out, same values bit for bit), without the pass-1
 * epilogue: for callers that run pass 1 themselves (qb_margins_topk) or
 * only need the scores.  Same layouts and limits.
 */
QB_API int qb_router_scores(const uint16_t* hidden, const uint16_t* w, int64_t N, int H, int E,
                            float* s_out, float* logits_out, qb_stream_t stream);

/*
 * Top-K expert loads per microbatch, for the local-balance metric
 * ("Exact Quantile Balancing and Load-Error Injection for Mixture-of-Experts",
 * summary page, background paragraph: global balance over all tokens of a
 * step, local balance inside each microbatch).  Each layer's N tokens are cut
 * into C = N / n_mb consecutive microbatches; load_mb[l][c][e] += number of
 * tokens of microbatch c whose top-K set of s + b[l] (ties: lower expert
 * index) contains e.  This is qb_margins_topk's load counting run per
 * microbatch, with the layer's bias shared by its microbatches.
 *   s float [L][N][E]; b float [L][E]; n_mb >= 1 must divide N;
 *   alpha float [L][N] receives the same values qb_margins_topk writes;
 *   load_mb int32 [L][C][E], accumulated (+=).
 */
QB_API int qb_microbatch_loads(const float* s, const float* b, int L, int64_t N, int E, int K,
                               int64_t n_mb, float* alpha, int32_t* load_mb, qb_stream_t stream);

/*
 * qb_margins_topk with loads and, in the same pass, the per-microbatch loads
 * of qb_microbatch_loads (each top-K member of token i also adds 1 to
 * load_mb[l][i / n_mb][e], one device atomic per member): the global and
 * the local balance of a batch from one read of the scores.
 *   load int32 [L][E] and load_mb int32 [L][N/n_mb][E] required,
 *   accumulated (+=); hist_hi nullable; n_mb must divide N.
 */
QB_API int qb_margins_topk_mb(const float* s, const float* b, int L, int64_t N, int E, int K, float* alpha,
                              int32_t* load, int32_t* hist_hi, int64_t n_mb, int32_t* load_mb,
                              qb_stream_t stream);

/*
 * MaxVio ("Exact Quantile Balancing and Load-Error Injection for
 * Mixture-of-Experts", summary page, testbed paragraph: how far the busiest
 * expert of the worst layer exceeds the uniform load).  For each of the L*C
 * rows of load (layer l, microbatch c; C = 1 for the whole batch), over
 * n_tok tokens each:
 *   maxvio[l][c] = fl32((double)max_e load[l][c][e] / ((double)n_tok * K / E) - 1)
 *   summary[l]   = {max over c, fl32(float64 sum over c in order / C)}  (nullable)
 *   worst        = {max over l of summary[l][0], max over l of summary[l][1]}  (nullable)
 *   load int32 [L][C][E]; maxvio float [L][C]; summary float [L][2]; worst float [2].
 *   Any E >= 1, 1 <= K <= E, n_tok >= 1.
 */
QB_API int qb_maxvio(const int32_t* load, int L, int C, int E, int K, int64_t n_tok, float* maxvio,
                     float* summary, float* worst, qb_stream_t stream);

/*
 * LEI per local batch, optionally bounded, and the gradient through the
 * router sigmoid ("Exact Quantile Balancing and Load-Error Injection for
 * Mixture-of-Experts", summary page, LEI paragraph: each token of a local
 * batch gets eta * rho_e added to its gradient for expert e's score; the
 * page's "normalized" variant limits the size of the residual vector with
 * tanh while leaving its direction and its zero sum unchanged, without
 * printing a formula -- the scaling used here is the simplest one with
 * those properties).  The N rows
 * form C = N / n_mb microbatches of n_mb rows; for microbatch c:
 *   rho_e  = fl32(((double)load_mb[c][e] - M) / M),  M = n_mb * K / E
 *   bounded == 1: rho_e = fl32((double)rho_e * tanh(|rho|) / |rho|), |rho| =
 *            float64 L2 norm over the E experts (sum in expert order)
 *   add_e  = fl32(eta * rho_e);  g' = fl32(g + add_e)
 *   dlogit = fl32(g' * fl32(s * fl32(1 - s)))      (sigmoid derivative)
 * With n_mb = N and bounded = 0, g' is exactly qb_lei_grad's result.
 *   g float [N][E] (read); s float [N][E] (needed for dlogits);
 *   load_mb int32 [C][E]; g_out float [N][E] (nullable; may be g);
 *   dlogits float [N][E] (nullable); float arrays 16-byte aligned;
 *   C <= 65535.
 */
QB_API int qb_lei_backward(const float* g, const float* s, const int32_t* load_mb, int64_t N, int E, int K,
                           int64_t n_mb, float eta, int bounded, float* g_out, float* dlogits,
                           qb_stream_t stream);

/*
 * One-GPU emulation of data-parallel ranks ("Exact Quantile Balancing and
 * Load-Error Injection for Mixture-of-Experts", summary page, background
 * paragraph: rank-local quantiles averaged across ranks depend on the
 * sharding, a histogram summed over ranks does not; EQB paragraph: two
 * all-reduces of byte histograms per update).  R emulated ranks keep their
 * copies of a per-rank buffer back to back, rank r's M elements at r * M.
 *
 * qb_allreduce_sum_i32: every rank's copy becomes the elementwise sum of all
 * R copies (an all-reduce of int32 counts).  buf int32 [R][M], in place.
 */
QB_API int qb_allreduce_sum_i32(int32_t* buf, int R, int64_t M, qb_stream_t stream);

/*
 * qb_rank_average: the rank-averaged update of the MARIN implementation the
 * same paragraph describes.  From rank-local quantiles q float [R][E]:
 *   qbar_j = fl32(sum_r (double)q[r][j] / R)            (rank order)
 *   b[j]   = fl32((double)qbar_j - mean_j (double)qbar_j) (float64 sum in expert order / E)
 *   bounds = {fl32(min b - 1), fl32(max b + 1)}          (nullable)
 * b float [E]; bounds float [2].  1 <= E <= 16384.
 */
QB_API int qb_rank_average(const float* q, int R, int E, float* b, float* bounds, qb_stream_t stream);

/*
 * LEI ("Exact Quantile Balancing and Load-Error Injection for
 * Mixture-of-Experts", summary page, LEI paragraph): with M = N*K/E,
 * rho_e = fl32((load_e - M) / M) in float64, add_e = fl32(eta * rho_e),
 * g[i][e] = fl32(g[i][e] + add_e) for every token i.  g: float [N][E] in/out
 * (16-byte aligned); load: int32 [E].
 */
QB_API int qb_lei_grad(float* g, const int32_t* load, int64_t N, int E, int K, float eta,
                       qb_stream_t stream);

/* Short name of a status code (static storage). */
QB_API const char* qb_status_string(int status);

/* Detailed message of this thread's last failed call ("" if none). */
QB_API const char* qb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QB_H */
