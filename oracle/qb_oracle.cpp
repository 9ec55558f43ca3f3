// qb_oracle.cpp -- CPU oracle for the quantile-balancing (QB) bias update.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, single-threaded,
// obviously-correct definition that the GPU library is checked against.  Only
// the test suite, the smoke check and the benchmark's CPU-baseline leg may load
// it.  It shares no source, header, table or helper with the HIP library, and
// the library never calls it.
//
// Sources (cited by page title and section):
//   [PR]  "[Dev] Add global-batch quantile balancing", Megatron-LM pull
//         request #6637: sections "Quantile estimator" (alpha, margin,
//         quantile, mean-centring, K3 histogram range and 1000 bins),
//         "Implementation" (int32 histogram [experts, bins] accumulated over
//         microbatches; FP32 bias and bounds updated in place), and the review
//         thread (total tokens read from expert 0's histogram row, valid
//         because every token adds one margin per expert).
//   [EQB] "Exact Quantile Balancing and Load-Error Injection for
//         Mixture-of-Experts" (paper summary page): the EQB paragraph (bf16
//         margins, two 256-bin byte histograms, the bin holding the rank),
//         the background paragraph (QB = K/E quantile of the margins) and the
//         LEI paragraph (expert e's score gradient shifted by eta * rho_e).
//
// Readings of points the pages leave open (each is a stated convention):
//   * rank: the quantile at level K/E of N margins is the order statistic of
//     1-based rank m = ceil(K*N/E) (inverse empirical CDF).
//   * "(k+1)-th largest" counts duplicates; values are ordered by IEEE-754
//     totalOrder (so +0 ranks above -0), ties of equal bit patterns broken by
//     the lower expert index.  The top-K set (for per-expert loads) is the
//     first K of that same order.
//   * margin r = fl32(alpha - s) with the raw score s; bf16 rounding is
//     round-to-nearest, ties-to-even, no flush of subnormals.
//   * order-preserving 16-bit key of a bf16 pattern u: negative -> ~u,
//     non-negative -> u | 0x8000.
//   * mean: float64 sum in expert order, divided by E, subtracted in float64,
//     rounded once to float32.  Bounds: [fl32(min - 1), fl32(max + 1)].
//   * K3 bins: fp32 margin (no bf16 rounding), bin = floor(fl32(fl32(r - lo)
//     * fl32(n_bins / fl32(hi - lo)))) clamped to [0, n_bins - 1]; the pooled
//     quantile is read by linear interpolation inside the bin holding rank m,
//     in float64.  (Which in-bin estimate K3 uses is not printed: parity
//     unpinned against the pages; pinned only by containment in that bin.)
//   * LEI: rho_e = (load_e - M) / M with M = N*K/E (float64, rounded to fp32),
//     add_e = fl32(eta * rho_e), g[i][e] = fl32(g[i][e] + add_e); unbounded.
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fPIC -shared (no fast-math).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

uint32_t f32_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return u;
}

float bits_f32(uint32_t u) {
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

// Value of a bf16 pattern, widened exactly to float.
float bf16_value(uint16_t u) { return bits_f32(uint32_t(u) << 16); }

// Round a float to the nearest bf16, ties to the even pattern, by the
// definition: take the two bf16 neighbours of x that bracket it (truncation
// toward zero and the next pattern away from zero) and keep the nearer one.
// Distances are exact in double.  Magnitudes past the largest finite bf16 use
// 2^128 as the upper neighbour (IEEE overflow rule), so they round to inf
// only from the halfway point on.  NaN is outside the domain.
uint16_t bf16_rne(float x) {
  const uint32_t bits = f32_bits(x);
  const uint16_t t = uint16_t(bits >> 16);
  const double dx = double(x);
  const double lo = double(bf16_value(t));
  if (lo == dx) return t;
  const uint16_t t2 = uint16_t(t + 1);
  const double hi = ((t2 & 0x7FFFu) == 0x7F80u) ? std::copysign(std::ldexp(1.0, 128), dx)
                                                 : double(bf16_value(t2));
  const double d_lo = std::fabs(dx - lo);
  const double d_hi = std::fabs(hi - dx);
  if (d_lo < d_hi) return t;
  if (d_hi < d_lo) return t2;
  return (t & 1u) == 0 ? t : t2;
}

// Order-preserving map of a bf16 pattern to an unsigned 16-bit key.
uint16_t key_of(uint16_t u) { return (u & 0x8000u) ? uint16_t(~u) : uint16_t(u | 0x8000u); }
uint16_t unkey(uint16_t k) { return (k & 0x8000u) ? uint16_t(k & 0x7FFFu) : uint16_t(~k); }

struct Scored {
  float v;
  int j;
};

// "a ranks before b": larger value first under IEEE totalOrder, then the
// lower expert index.
bool ranks_before(const Scored& a, const Scored& b) {
  if (a.v > b.v) return true;
  if (a.v < b.v) return false;
  const bool na = std::signbit(a.v), nb = std::signbit(b.v);
  if (na != nb) return !na;  // +0 ranks above -0
  return a.j < b.j;
}

int64_t rank_m(int64_t N, int E, int K) { return (int64_t(K) * N + E - 1) / E; }

// [PR, Quantile estimator]: b_next -= mean(b_next); next bounds
// [min(b_next) - 1, max(b_next) + 1].
void centre_and_bounds(const float* q, int E, float* b_next, float* bounds) {
  double sum = 0.0;
  for (int j = 0; j < E; ++j) sum += double(q[j]);
  const double mean = sum / double(E);
  for (int j = 0; j < E; ++j) b_next[j] = float(double(q[j]) - mean);
  float mn = b_next[0], mx = b_next[0];
  for (int j = 1; j < E; ++j) {
    if (b_next[j] < mn) mn = b_next[j];
    if (b_next[j] > mx) mx = b_next[j];
  }
  bounds[0] = mn - 1.0f;
  bounds[1] = mx + 1.0f;
}

}  // namespace

extern "C" {

uint16_t oq_bf16_rne(float x) { return bf16_rne(x); }
float oq_bf16_value(uint16_t u) { return bf16_value(u); }
uint16_t oq_key(uint16_t u) { return key_of(u); }
uint16_t oq_unkey(uint16_t k) { return unkey(k); }

void oq_bf16_rne_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(x[i]);
}

// [PR, Quantile estimator]: alpha[i] = (K+1)-th largest of s[i,:] + b[:].
// load (nullable): += 1 for each expert in the first K of the order.
void oq_alpha(const float* s, const float* b, int64_t N, int E, int K, float* alpha,
              int32_t* load) {
  std::vector<Scored> row(E);
  for (int64_t i = 0; i < N; ++i) {
    for (int j = 0; j < E; ++j) row[j] = Scored{s[i * E + j] + b[j], j};
    std::partial_sort(row.begin(), row.begin() + (K + 1), row.end(), ranks_before);
    alpha[i] = row[K].v;
    if (load)
      for (int k = 0; k < K; ++k) load[row[k].j] += 1;
  }
}

// 16-bit keys of the bf16-rounded margins r = fl32(alpha_i - s_ij), written
// expert-major: keys_t[j * N + i].
void oq_margin_keys(const float* s, const float* alpha, int64_t N, int E, uint16_t* keys_t) {
  for (int64_t i = 0; i < N; ++i)
    for (int j = 0; j < E; ++j) {
      const float r = alpha[i] - s[i * E + j];
      keys_t[int64_t(j) * N + i] = key_of(bf16_rne(r));
    }
}

// One layer of EQB.  The quantile is found by sorting each expert's N keys and
// picking position m-1; the radix intermediates are recomputed by direct
// counting so the GPU's two histogram passes can be compared element by
// element:
//   hist_hi[j][h]  = #{i : key_ij >> 8 == h}
//   sel_hi[j]      = key*_j >> 8           (taken from the sort)
//   rank_lo[j]     = m - #{i : key_ij >> 8 < sel_hi[j]}
//   hist_lo[j][l]  = #{i : key_ij >> 8 == sel_hi[j] and key_ij & 0xFF == l}
//   key_star[j]    = sorted keys of expert j at position m-1
//   q[j]           = value of the bf16 pattern behind key_star[j]
// [EQB, EQB paragraph]; [PR, Quantile estimator].  Returns 0.
int oq_eqb_layer(const float* s, const float* b, int64_t N, int E, int K, float* alpha,
                 int32_t* load, int32_t* hist_hi, int32_t* sel_hi, int32_t* rank_lo,
                 int32_t* hist_lo, uint16_t* key_star, float* q, float* b_next, float* bounds) {
  oq_alpha(s, b, N, E, K, alpha, load);
  std::vector<uint16_t> keys_t(size_t(N) * size_t(E));
  oq_margin_keys(s, alpha, N, E, keys_t.data());
  const int64_t m = rank_m(N, E, K);
  std::memset(hist_hi, 0, sizeof(int32_t) * size_t(E) * 256);
  std::memset(hist_lo, 0, sizeof(int32_t) * size_t(E) * 256);
  for (int j = 0; j < E; ++j) {
    uint16_t* col = keys_t.data() + int64_t(j) * N;
    int32_t* hh = hist_hi + int64_t(j) * 256;
    for (int64_t i = 0; i < N; ++i) hh[col[i] >> 8] += 1;
    std::sort(col, col + N);
    const uint16_t ks = col[m - 1];
    key_star[j] = ks;
    q[j] = bf16_value(unkey(ks));
    const int h = ks >> 8;
    sel_hi[j] = h;
    int64_t below = 0;
    for (int hb = 0; hb < h; ++hb) below += hh[hb];
    rank_lo[j] = int32_t(m - below);
    int32_t* hl = hist_lo + int64_t(j) * 256;
    for (int64_t i = 0; i < N; ++i)
      if ((col[i] >> 8) == h) hl[col[i] & 0xFF] += 1;
  }
  centre_and_bounds(q, E, b_next, bounds);
  return 0;
}

// K3 bin of an fp32 margin (see the header for the reading).
int oq_k3_bin(float r, float lo, float hi, int n_bins) {
  const float width = hi - lo;
  const float inv_w = float(n_bins) / width;
  const float t = (r - lo) * inv_w;
  if (!(t >= 0.0f)) return 0;
  if (t >= float(n_bins)) return n_bins - 1;
  return int(t);
}

// One layer of K3: alpha as above, n_bins uniform bins per expert over the
// current bounds [lo, hi] of the fp32 margins, then the pooled quantile read
// from each expert's histogram at rank m by linear interpolation inside the
// bin that holds it, mean-centred; bounds_out = next batch's range.
// [PR, Quantile estimator; Implementation].  Returns 0, or -1 if a row never
// reaches rank m (impossible for a well-formed histogram).
int oq_k3_layer(const float* s, const float* b, int64_t N, int E, int K, const float* bounds_in,
                int n_bins, float* alpha, int32_t* hist_u, float* q, float* b_next,
                float* bounds_out) {
  oq_alpha(s, b, N, E, K, alpha, nullptr);
  const float lo = bounds_in[0], hi = bounds_in[1];
  std::memset(hist_u, 0, sizeof(int32_t) * size_t(E) * size_t(n_bins));
  for (int64_t i = 0; i < N; ++i)
    for (int j = 0; j < E; ++j) {
      const float r = alpha[i] - s[i * E + j];
      hist_u[int64_t(j) * n_bins + oq_k3_bin(r, lo, hi, n_bins)] += 1;
    }
  const int64_t m = rank_m(N, E, K);
  const double w = (double(hi) - double(lo)) / double(n_bins);
  for (int j = 0; j < E; ++j) {
    const int32_t* h = hist_u + int64_t(j) * n_bins;
    int64_t before = 0;
    int c = 0;
    while (c < n_bins && before + h[c] < m) before += h[c++];
    if (c == n_bins) return -1;
    const double frac = double(m - before) / double(h[c]);
    q[j] = float(double(lo) + w * (double(c) + frac));
  }
  centre_and_bounds(q, E, b_next, bounds_out);
  return 0;
}

// Next-batch K3 range from a bias vector: [fl32(min b - 1), fl32(max b + 1)].
void oq_bounds_of(const float* b, int E, float* bounds) {
  float mn = b[0], mx = b[0];
  for (int j = 1; j < E; ++j) {
    if (b[j] < mn) mn = b[j];
    if (b[j] > mx) mx = b[j];
  }
  bounds[0] = mn - 1.0f;
  bounds[1] = mx + 1.0f;
}

// [EQB, LEI paragraph]: the gradient of every token with respect to expert
// e's score is shifted by eta * rho_e, rho_e = relative load error of e.
void oq_lei(float* g, const int32_t* load, int64_t N, int E, int K, float eta) {
  const double M = double(N) * double(K) / double(E);
  std::vector<float> add(E);
  for (int e = 0; e < E; ++e) {
    const float rho = float((double(load[e]) - M) / M);
    add[e] = eta * rho;
  }
  for (int64_t i = 0; i < N; ++i)
    for (int e = 0; e < E; ++e) g[i * E + e] = g[i * E + e] + add[e];
}

// LEI per microbatch ([EQB] LEI paragraph: the shift eta * rho_e applies to
// every token of the local batch), optionally with the bounded
// ("normalized") residual -- its size limited by tanh, its direction and
// zero sum kept; no formula is printed, so this reading (rho scaled by
// tanh(|rho|) / |rho|, L2 norm in float64) is parity unpinned against the
// pages -- and the gradient through the sigmoid:
//   g' = fl32(g + fl32(eta * rho_e)), dlogit = fl32(g' * fl32(s * fl32(1 - s))).
// g_out and dlogits may be NULL.
void oq_lei_bwd(const float* g, const float* s, const int32_t* load_mb, int64_t N, int E, int K, int64_t n_mb,
                float eta, int bounded, float* g_out, float* dlogits) {
  const double M = double(n_mb) * double(K) / double(E);
  std::vector<float> rho(E), add(E);
  for (int64_t c = 0; c < N / n_mb; ++c) {
    const int32_t* load = load_mb + c * E;
    for (int e = 0; e < E; ++e) rho[e] = float((double(load[e]) - M) / M);
    if (bounded) {
      double n2 = 0.0;
      for (int e = 0; e < E; ++e) n2 += double(rho[e]) * double(rho[e]);
      const double norm = std::sqrt(n2);
      const double lambda = norm > 0.0 ? std::tanh(norm) / norm : 1.0;
      for (int e = 0; e < E; ++e) rho[e] = float(double(rho[e]) * lambda);
    }
    for (int e = 0; e < E; ++e) add[e] = eta * rho[e];
    for (int64_t i = c * n_mb; i < (c + 1) * n_mb; ++i)
      for (int e = 0; e < E; ++e) {
        const int64_t k = i * E + e;
        const float gp = g[k] + add[e];
        if (g_out) g_out[k] = gp;
        if (dlogits) {
          const float one_minus = 1.0f - s[k];
          const float ds = s[k] * one_minus;
          dlogits[k] = gp * ds;
        }
      }
  }
}

// Router logits of selected rows, bf16 inputs, float64 accumulation; the
// weight is stored [E][H] (nn.Linear layout):
// out[r * E + e] = sum_h hidden[rows[r]][h] * w[e][h].
void oq_router_logits(const uint16_t* hidden, const uint16_t* w, int H, int E,
                      const int64_t* rows, int n_rows, double* out) {
  for (int r = 0; r < n_rows; ++r) {
    const uint16_t* x = hidden + rows[r] * int64_t(H);
    for (int e = 0; e < E; ++e) {
      const uint16_t* we = w + int64_t(e) * H;
      double acc = 0.0;
      for (int h = 0; h < H; ++h) acc += double(bf16_value(x[h])) * double(bf16_value(we[h]));
      out[int64_t(r) * E + e] = acc;
    }
  }
}

// Rank-averaged update ([EQB] background paragraph: the MARIN
// implementation averages rank-local quantiles across data-parallel ranks):
// qbar_j = fl32(sum_r (double)q[r][j] / R) in rank order, then the same
// centring and bounds as the EQB update.
void oq_rank_average(const float* q, int R, int E, float* b, float* bounds) {
  std::vector<float> qbar(E);
  for (int j = 0; j < E; ++j) {
    double sum = 0.0;
    for (int r = 0; r < R; ++r) sum += double(q[int64_t(r) * E + j]);
    qbar[j] = float(sum / double(R));
  }
  double sum = 0.0;
  for (int j = 0; j < E; ++j) sum += double(qbar[j]);
  const double mean = sum / double(E);
  for (int j = 0; j < E; ++j) b[j] = float(double(qbar[j]) - mean);
  oq_bounds_of(b, E, bounds);
}

// MaxVio ([EQB] testbed paragraph: how far the busiest expert exceeds the
// uniform load; background paragraph: global vs per-microbatch balance).
// Rows are (layer, microbatch) pairs of E loads over n_tok tokens each:
//   v[r] = fl32(max_e load[r][e] / (n_tok * K / E) - 1) in float64;
// per layer: summary = {max over its C rows, fl32(float64 sum / C)};
// worst = {max over layers of each}.  summary / worst may be NULL.
void oq_maxvio(const int32_t* load, int L, int C, int E, int K, int64_t n_tok, float* v,
               float* summary, float* worst) {
  const double share = double(n_tok) * double(K) / double(E);
  float wmax = -INFINITY, wmean = -INFINITY;
  for (int l = 0; l < L; ++l) {
    float mx = -INFINITY;
    double sum = 0.0;
    for (int c = 0; c < C; ++c) {
      const int32_t* row = load + (int64_t(l) * C + c) * E;
      int32_t m = row[0];
      for (int e = 1; e < E; ++e) m = std::max(m, row[e]);
      const float vi = float(double(m) / share - 1.0);
      v[int64_t(l) * C + c] = vi;
      mx = std::max(mx, vi);
      sum += double(vi);
    }
    const float mean = float(sum / double(C));
    if (summary) {
      summary[2 * l] = mx;
      summary[2 * l + 1] = mean;
    }
    wmax = std::max(wmax, mx);
    wmean = std::max(wmean, mean);
  }
  if (worst) {
    worst[0] = wmax;
    worst[1] = wmean;
  }
}

}  // extern "C"
