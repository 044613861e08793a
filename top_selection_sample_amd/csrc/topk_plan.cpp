// Host-side parameter selection for the sampled threshold, and the plan of a
// call shape (route, buffer capacity, launch shapes, workspace layout).
//
// Algorithm 1 of the Prof-K paper ("Adaptive parameter selection"):
//   z = 2 * Phi^-1(1 - eps/2);  alpha = k/N
//   S* = (z * (tau_B/tau_A) * log2 k / 2)^(2/3) * (k (N-k))^(1/3)   (Eq. 14)
//   S = clamp(round(S*), S_min, S_max);  f = 1 - S/N
//   t = max(1, ceil(S alpha + z/2 sqrt(S alpha (1-alpha) f)))     (Eq. 6)
//   M = ceil(k + z sqrt(k (N-k) f / S))                           (Eq. 12)
//   t = 1 when alpha S < -ln(eps/2)
//
// Default policy ("exact tail"): S as above; t and M the least values that
// meet Theorem 3's two conditions with eps_A = eps_B = eps/2, using the exact
// law of the threshold rank (Lemma 1): with H(N, K, S) the number of sampled
// items among K fixed items,
//   P(R < k) = P(H(N, k-1, S) >= t),   P(R > M) = P(H(N, M, S) <= t-1).
//
// Tuned policy: t and M as in the exact-tail policy, and S the minimiser of
// Eq. 13's overhead C(S) = tau_A S + tau_B M(S) log2 k with the exact-tail
// M(S), over a quarter-octave grid of sample sizes, with tau_B / tau_A
// measured on this engine.  The lower bound S_min of Algorithm 1 guards the
// normal approximation; the exact tail needs no such guard, so the grid
// starts lower.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "topk_launch.hpp"
#include "topk_plan.hpp"

namespace tk {

// Inverse of the standard normal CDF by bisection on 0.5*erfc(-x/sqrt 2).
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    const double c = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (c < p) lo = mid;
    else hi = mid;
  }
  return 0.5 * (lo + hi);
}

Alg1 algorithm1(int64_t N, int64_t k, double eps, int64_t s_min, int64_t s_max, double ratio) {
  Alg1 a;
  const double zq = normal_quantile(1.0 - eps / 2.0);
  a.z = zq + zq;
  const double Nd = (double)N, kd = (double)k;
  const double alpha = kd / Nd;
  a.s_star = std::pow(a.z * ratio * std::log2(kd) / 2.0, 2.0 / 3.0) *
             std::cbrt(kd * (Nd - kd));
  int64_t S = (int64_t)std::floor(a.s_star + 0.5);
  if (S < s_min) S = s_min;
  if (S > s_max) S = s_max;
  if (S > N) S = N;   // stage 1 draws S of the N items without replacement
  a.S = S;
  const double Sd = (double)S;
  const double f = 1.0 - Sd / Nd;
  double tt = std::ceil(Sd * alpha + a.z / 2.0 * std::sqrt(std::fmax(0.0, Sd * alpha * (1 - alpha) * f)));
  a.t = tt < 1.0 ? 1 : (int64_t)tt;
  a.M = (int64_t)std::ceil(kd + a.z * std::sqrt(std::fmax(0.0, kd * (Nd - kd) / Sd * f)));
  if (alpha * Sd < -std::log(eps / 2.0)) a.t = 1;
  return a;
}

// ---------------------------------------------------------------- hypergeometric
namespace {

double log_binom(double a, double b) {
  return std::lgamma(a + 1.0) - std::lgamma(b + 1.0) - std::lgamma(a - b + 1.0);
}

// log P(H = j_min) with j_min = max(0, S - (N - K)).  When j_min = 0 it is the
// product prod_{i<m} (1 - a/(N - i)) over the smaller m of (K, S), summed as
// log1p terms (accurate); `fast` uses lgamma instead (about 1e-6 relative).
double log_p_first(int64_t N, int64_t K, int64_t S, int64_t* j_min, bool fast) {
  const int64_t jm = (S - (N - K)) > 0 ? (S - (N - K)) : 0;
  *j_min = jm;
  if (jm > 0 || fast)
    return log_binom((double)K, (double)jm) + log_binom((double)(N - K), (double)(S - jm)) -
           log_binom((double)N, (double)S);
  const int64_t m = K < S ? K : S;
  const double a = (double)(K < S ? S : K);
  double s = 0.0, c = 0.0;  // Kahan sum
  for (int64_t i = 0; i < m; ++i) {
    const double y = std::log1p(-a / (double)(N - i)) - c;
    const double t = s + y;
    c = (t - s) - y;
    s = t;
  }
  return s;
}

// log P(j+1) - log P(j)
inline double log_ratio(int64_t N, int64_t K, int64_t S, int64_t j) {
  return std::log((double)(K - j) * (double)(S - j)) -
         std::log((double)(j + 1) * (double)(N - K - S + j + 1));
}

}  // namespace

double hyper_cdf(int64_t N, int64_t K, int64_t S, int64_t t, bool fast) {
  if (t < 0) return 0.0;
  int64_t j;
  double lp = log_p_first(N, K, S, &j, fast);
  const int64_t hi = K < S ? K : S;
  double sum = 0.0;
  for (; j <= t && j <= hi; ++j) {
    sum += std::exp(lp);
    if (j < hi) lp += log_ratio(N, K, S, j);
  }
  return sum;
}

double hyper_sf(int64_t N, int64_t K, int64_t S, int64_t t) {
  const int64_t hi = K < S ? K : S;
  if (t > hi) return 0.0;
  int64_t j;
  double lp = log_p_first(N, K, S, &j, false);
  if (t <= j) return 1.0;
  for (; j < t; ++j) lp += log_ratio(N, K, S, j);
  const double mode = (double)(K + 1) * (double)(S + 1) / (double)(N + 2);
  double sum = 0.0;
  for (;; ++j) {
    const double p = std::exp(lp);
    sum += p;
    if (j >= hi || ((double)j > mode && p < sum * 1e-18)) break;
    lp += log_ratio(N, K, S, j);
  }
  return sum;
}

TailParams exact_tail(int64_t N, int64_t k, int64_t S, double eps) {
  TailParams r;
  const double half = eps / 2.0;
  // t: least t >= 1 with P(H(N, k-1, S) >= t) <= eps/2.  The pmf is walked
  // once from its first support point; the upper tail is a suffix sum.
  int64_t t = 1;
  if (k > 1) {
    const int64_t K = k - 1, hi = K < S ? K : S;
    int64_t j0;
    double lp = log_p_first(N, K, S, &j0, false);
    const double mode = (double)(K + 1) * (double)(S + 1) / (double)(N + 2);
    std::vector<double> pm;
    double tot = 0.0;
    for (int64_t j = j0;; ++j) {
      const double p = std::exp(lp);
      pm.push_back(p);
      tot += p;
      if (j >= hi || ((double)j > mode && p < tot * 1e-18)) break;
      lp += log_ratio(N, K, S, j);
    }
    // suffix sums: sf[j - j0] = P(H >= j)
    std::vector<double> sf(pm.size() + 1, 0.0);
    for (int64_t i = (int64_t)pm.size() - 1; i >= 0; --i) sf[i] = sf[i + 1] + pm[i];
    auto tail = [&](int64_t tt) -> double {
      if (tt <= j0) return 1.0;
      const int64_t i = tt - j0;
      return i < (int64_t)sf.size() ? sf[i] : 0.0;
    };
    while (t < S && tail(t) > half) ++t;
  }
  r.t = t;
  int64_t M;
  if (hyper_cdf(N, N, S, t - 1, true) > half) {
    M = N;
  } else {
    int64_t lo = k, hi = N;
    while (lo < hi) {  // least M with P(R > M) <= eps/2 (lgamma form)
      const int64_t mid = lo + (hi - lo) / 2;
      if (hyper_cdf(N, mid, S, t - 1, true) <= half) hi = mid;
      else lo = mid + 1;
    }
    M = lo;
    // settle the boundary with the accurate form
    while (M < N && hyper_cdf(N, M, S, t - 1, false) > half) ++M;
    while (M > k && hyper_cdf(N, M - 1, S, t - 1, false) <= half) --M;
  }
  r.M = M;
  return r;
}

// Quarter-octave grid s_lo * 2^(j/4), j = 0, 1, ... up to s_hi; the point
// with the least C(S) / tau_A = S + ratio * M(S) * log2 k wins (the smaller S
// on a tie).
int64_t tuned_sample_size(int64_t N, int64_t k, double eps, int64_t s_lo, int64_t s_hi,
                          double ratio) {
  if (s_lo > N) s_lo = N;
  if (s_hi > N) s_hi = N;
  if (s_hi < s_lo) return s_lo;
  const double lk = std::log2((double)k);
  int64_t best = s_lo;
  double best_c = 0.0;
  int64_t prev = 0;
  for (int j = 0;; ++j) {
    int64_t S = (int64_t)std::llround((double)s_lo * std::exp2(0.25 * j));
    if (S > s_hi) break;
    if (S == prev) continue;
    prev = S;
    const TailParams tp = exact_tail(N, k, S, eps);
    const double c = (double)S + ratio * (double)tp.M * lk;
    if (j == 0 || c < best_c) {
      best = S;
      best_c = c;
    }
  }
  return best;
}

// ---------------------------------------------------------------- cache
namespace {
struct Key {
  int64_t N, k, s_min, s_max, S, t, M, tuned_s_min;
  double eps, ratio, tuned_ratio;
  int policy;
  bool operator<(const Key& o) const {
    return std::tie(N, k, s_min, s_max, S, t, M, tuned_s_min, eps, ratio, tuned_ratio, policy) <
           std::tie(o.N, o.k, o.s_min, o.s_max, o.S, o.t, o.M, o.tuned_s_min, o.eps, o.ratio,
                    o.tuned_ratio, o.policy);
  }
};
struct Val {
  int64_t S, t, M;
  double pr, po;
};
std::mutex g_mu;
std::map<Key, Val> g_cache;

uint32_t bitlen(uint64_t v) {
  uint32_t b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

void sample_params(int64_t N, int64_t k, const ParamIn& in, int64_t* S, int64_t* t, int64_t* M,
                   double* pr, double* po) {
  const double tratio = k > KSMALL ? in.tuned_ratio_large : in.tuned_ratio;
  Key key{N,      k,     in.s_min,      in.s_max,       in.S,      in.t,
          in.M,   in.tuned_s_min, in.eps, in.cost_ratio, tratio, in.policy};
  {
    std::lock_guard<std::mutex> g(g_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) {
      *S = it->second.S;
      *t = it->second.t;
      *M = it->second.M;
      *pr = it->second.pr;
      *po = it->second.po;
      return;
    }
  }
  const Alg1 a = algorithm1(N, k, in.eps, in.s_min, in.s_max, in.cost_ratio);
  int64_t s = a.S;
  if (in.S > 0) s = in.S;
  else if (in.policy == 2)
    s = tuned_sample_size(N, k, in.eps, in.tuned_s_min, std::min(in.s_max, N / 8), tratio);
  if (s > N) s = N;
  int64_t tt, mm;
  if (in.policy == 1) {
    tt = a.t;
    mm = a.M;
  } else {
    const TailParams tp = exact_tail(N, k, s, in.eps);
    tt = tp.t;
    mm = tp.M;
  }
  if (in.t > 0) tt = in.t;
  if (in.M > 0) mm = in.M;
  if (tt > s) tt = s;
  if (mm > N) mm = N;
  const double prv = (k > 1) ? hyper_sf(N, k - 1, s, tt) : 0.0;
  const double pov = hyper_cdf(N, mm, s, tt - 1, false);
  {
    std::lock_guard<std::mutex> g(g_mu);
    g_cache[key] = Val{s, tt, mm, prv, pov};
  }
  *S = s;
  *t = tt;
  *M = mm;
  *pr = prv;
  *po = pov;
}

int make_plan(int64_t n, int64_t rows, int64_t k, int dtype, const ParamIn& in, Plan* out) {
  Plan p;
  p.n = n;
  p.rows = rows;
  p.k = k;
  p.dtype = dtype;
  p.KB = (dtype == 2) ? 16u : 32u;
  const uint32_t bl = bitlen((uint64_t)n);      // 2^B > n, so every index field is >= 1
  p.B = ((bl + 7u) / 8u) * 8u;
  if (p.B < 8) p.B = 8;
  p.W = p.KB + p.B;
  uint32_t b = bitlen((uint64_t)(n - 1));       // 2^b >= n
  if (b < 2) b = 2;
  p.half_bits = (b + 1u) / 2u;
  p.small_k = k <= KSMALL;

  // eps bounds the fallback probability of the whole call: the rows of a
  // batch are independent selections, so each gets eps / rows (Algorithm 1
  // verbatim keeps its per-selection eps)
  ParamIn row_in = in;
  if (rows > 1 && in.policy != 1) row_in.eps = in.eps / (double)rows;
  // relaxed recall: the parameters are those of the smaller selection
  // k_eff = ceil(recall * k) (a row keeps its survivors once it has k_eff)
  p.k_eff = k;
  if (in.recall < 1.0) {
    p.k_eff = (int64_t)std::ceil(in.recall * (double)k - 1e-9);
    if (p.k_eff < 1) p.k_eff = 1;
    if (p.k_eff > k) p.k_eff = k;
  }
  // the refine that runs is the one for k: its cost ratio prices the buffer
  if (k > KSMALL) row_in.tuned_ratio = in.tuned_ratio_large;
  else if (rows >= in.tuned_batch_rows) row_in.tuned_ratio = in.tuned_ratio_batched;
  sample_params(n, p.k_eff, row_in, &p.S, &p.t, &p.M, &p.p_recall, &p.p_overflow);
  const int es = (dtype == 2) ? 2 : 4;
  const int64_t cus = in.cus > 0 ? in.cus : 256;
  // Rows up to EXACT_SMALL_MAX can instead be selected one workgroup per
  // row, exactly and with no sample.  Measured on MI355X, that costs about
  // 8 us + 0.84 ns per element for each round of rows (one row per compute
  // unit), and the sampled route about 22 us + 0.025 us per row + the input
  // read at 7 TB/s; the cheaper one runs.  (One row of 2^16 elements: 64 us
  // in one workgroup, 21 us sampled; one row of 4096: 12 against 22.)
  bool small_cheaper = false;
  if (n <= EXACT_SMALL_MAX) {
    const double rounds = (double)((rows + cus - 1) / cus);
    const double t_small = (8.0 + 8.4e-4 * (double)n) * rounds;
    const double t_sampled = 22.0 + 0.025 * (double)rows + (double)rows * (double)n * es / 7.0e6;
    small_cheaper = t_small <= t_sampled;
  }
  bool sampled;
  p.force_tau = in.force_tau;
  if (in.force_path == 1 || in.force_tau) sampled = true;
  else if (in.force_path == 2) sampled = false;
  else sampled = (n >= 8 * p.S) && (p.M < n / 2) && !small_cheaper;
  if (sampled) {
    p.path = PLAN_SAMPLED;
    p.cap = p.M < k ? k : p.M;
    if (p.cap > n) p.cap = n;
  } else if (n <= EXACT_SMALL_MAX) {
    p.path = PLAN_EXACT_SMALL;
    p.cap = k;
  } else {
    p.path = PLAN_EXACT;
    int64_t c = 2 * k > 16384 ? 2 * k : 16384;
    p.cap = c > n ? n : c;
  }
  // filter grid: one or two workgroups per compute unit over the whole call,
  // each a contiguous slice of one row no shorter than 64 KB.  With few
  // survivors one 512-thread workgroup per CU is faster (the next step's
  // loads are in flight while a step is examined; 2.5% on 2^28 fp32 at
  // t/S = 4e-5); with many (t/S ~ 1e-3: bf16 BatchTopK, 128 short rows) two
  // hide the survivor handling better (4% and 16% faster there)
  const bool dense = (double)p.t > 2e-4 * (double)p.S;
  int64_t fb = ((dense ? 2 : 1) * cus + rows / 2) / rows;
  const int64_t max_slices = (n * es) / 65536;
  if (fb > max_slices) fb = max_slices;
  if (fb < 1) fb = 1;
  p.filter_bpr = (uint32_t)fb;
  p.hist_bpr = 1;

  size_t off = 256;   // the workspace header (WsHeader)
  p.off_states = off;
  off = align256(off + (size_t)rows * 64);
  p.off_call = off;
  off = align256(off + 64);
  p.off_flag = off;
  off = align256(off + (size_t)rows * 4);
  p.off_ghist = off;
  if (p.path != PLAN_EXACT_SMALL) off = align256(off + (size_t)rows * 256 * 4);
  p.off_skeys = off;
  p.SP = (p.S + 3) / 4 * 4;   // sample-key rows padded for 16-byte loads
  if (p.path == PLAN_SAMPLED) off = align256(off + (size_t)rows * (size_t)p.SP * 4);
  p.off_shist = off;
  if (p.path == PLAN_SAMPLED) off = align256(off + (size_t)rows * 2048 * 4);

  p.off_cbuf = off;
  off = align256(off + (size_t)rows * (size_t)p.cap * 8);
  p.off_aux = off;   // large k: the merge buffer; sampled route: the tie region first
  if (!p.small_k || p.path == PLAN_SAMPLED) off = align256(off + (size_t)rows * (size_t)p.cap * 8);
  const bool lk = !p.small_k && p.cap <= LK_CAP_MAX;   // the bucket sort
  p.off_lkc = off;  // large k: per chunk, its prefix count by bucket rank
  if (lk) {
    const size_t chunks = (size_t)((p.cap + LK_CHUNK_CANDS - 1) / LK_CHUNK_CANDS);
    off = align256(off + (size_t)rows * chunks * LK_CSTRIDE * 4);
  }
  p.off_lks = off;  // large k: the split scratch
  if (lk) off = align256(off + (size_t)rows * (size_t)p.cap * 8);
  p.off_rctr = off;   // sampled route: four 128-byte counter lines per row
  if (p.path == PLAN_SAMPLED) off = align256(off + (size_t)rows * 512);
  p.total = off;
  // layout signature: every offset, the row count and the route
  uint64_t h = 0x9E3779B97F4A7C15ull;
  const uint64_t parts[] = {p.total,    p.off_states, p.off_call, p.off_flag, p.off_ghist,
                            p.off_skeys, p.off_shist, p.off_cbuf, p.off_aux,  p.off_lkc,
                            p.off_lks,   p.off_rctr,  (uint64_t)p.rows,
                            (uint64_t)p.path, (uint64_t)p.SP};
  for (uint64_t v : parts) h ^= v + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
  p.sig = h | 1ull;   // never 0
  *out = p;
  return 0;
}

}  // namespace tk
