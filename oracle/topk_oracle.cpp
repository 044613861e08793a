// CPU oracle for exact top-k selection.  TEST INFRASTRUCTURE ONLY: the test
// suite, the smoke check and the CPU-baseline leg of the benchmark may load
// this library; the product path never does.  It shares no code, header or
// constant with the HIP library.
//
// What it computes (plain definitions, written out):
//
//  * Problem (Prof-K paper, section 3 "Problem Setup"): return the k largest
//    entries of a row together with their indices; a batch applies the same
//    to every row.
//  * Order (GPU.js Learn "Rank by Counting", Goal and Hint 2): an element is
//    outranked by every strictly larger score and by every equal score at a
//    lower index.  Output slot r holds the element of rank r.
//  * Values are compared through order-preserving unsigned keys (a textbook
//    construction; the paper's related-work section mentions exploiting
//    float bit patterns).  Readings where the pages are silent: -0.0 and
//    +0.0 are the same value; every NaN is one value above +inf.
//  * Selection: a partial sort of the index array on (key desc, index asc);
//    the comparator is a strict total order, so the library's partial sort
//    returns exactly the first k in rank order.
//
//  * Sampler (paper section 3, stage 1 "Sampling"): S indices uniformly
//    without replacement.  Reading: the first S images of a keyed
//    pseudo-random permutation of [0, N): a 4-round balanced Feistel network
//    on 2h bits (2^(2h) >= N) whose round function is the SplitMix64 output
//    mixer (Steele, Lea & Flood, OOPSLA 2014), with cycle walking back into
//    [0, N) (Black & Rogaway, "Ciphers with arbitrary finite domains", 2002).
//    Round keys for (seed, row) are SplitMix64 outputs number 4*row .. 4*row+3
//    of the stream started at `seed`.
//  * Threshold (stage 2 "Threshold Estimation"): tau = the t-th largest
//    sampled key.  R = #{i : key_i >= tau} (the inclusive filter of stage 3).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

enum { OR_I32 = 0, OR_F32 = 1, OR_BF16 = 2 };

inline uint32_t key_i32(uint32_t bits) { return bits ^ 0x80000000u; }

inline uint32_t key_f32(uint32_t bits) {
  uint32_t mag = bits & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0xFFFFFFFFu;   // any NaN: above +inf
  if (mag == 0) return 0x80000000u;            // -0.0 is +0.0
  if (bits & 0x80000000u) return ~bits;        // negatives: reverse order
  return bits | 0x80000000u;                   // positives: above negatives
}

inline uint32_t key_bf16(uint16_t bits16) {
  uint32_t b = bits16;
  uint32_t mag = b & 0x7FFFu;
  if (mag > 0x7F80u) return 0xFFFFu;
  if (mag == 0) return 0x8000u;
  if (b & 0x8000u) return (~b) & 0xFFFFu;
  return b | 0x8000u;
}

int elem_size(int dtype) {
  switch (dtype) {
    case OR_I32: return 4;
    case OR_F32: return 4;
    case OR_BF16: return 2;
    default: return 0;
  }
}

uint32_t key_at(const unsigned char* base, int64_t i, int dtype) {
  if (dtype == OR_BF16) {
    uint16_t v;
    std::memcpy(&v, base + 2 * i, 2);
    return key_bf16(v);
  }
  uint32_t v;
  std::memcpy(&v, base + 4 * i, 4);
  return dtype == OR_I32 ? key_i32(v) : key_f32(v);
}

// SplitMix64 output mixer (the "mix64" finalizer of SplitMix64).
inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
// Output number j (0-based) of the SplitMix64 stream seeded with `seed`:
// the state advances by the golden-ratio increment before each output.
inline uint64_t sm64_output(uint64_t seed, uint64_t j) {
  return sm64_mix(seed + (j + 1) * 0x9E3779B97F4A7C15ull);
}

struct Perm {
  uint64_t n;
  uint32_t h;        // half width in bits
  uint64_t mask;     // (1 << h) - 1
  uint64_t rk[4];
};

Perm make_perm(uint64_t seed, uint64_t row, uint64_t n) {
  Perm p;
  p.n = n;
  uint32_t b = 0;
  while ((1ull << b) < n) ++b;     // 2^b >= n
  if (b < 2) b = 2;
  p.h = (b + 1) / 2;               // 2^(2h) >= 2^b >= n
  p.mask = (1ull << p.h) - 1;
  for (int r = 0; r < 4; ++r) p.rk[r] = sm64_output(seed, 4 * row + r);
  return p;
}

uint64_t feistel(const Perm& p, uint64_t x) {
  uint64_t L = x >> p.h, R = x & p.mask;
  for (int r = 0; r < 4; ++r) {
    uint64_t F = sm64_mix(R ^ p.rk[r]) & p.mask;
    uint64_t nl = R, nr = L ^ F;
    L = nl;
    R = nr;
  }
  return (L << p.h) | R;
}

uint64_t perm_index(const Perm& p, uint64_t i) {
  uint64_t x = feistel(p, i);
  while (x >= p.n) x = feistel(p, x);   // cycle walk; ends since i < n
  return x;
}

}  // namespace

extern "C" {

int oracle_elem_size(int dtype) { return elem_size(dtype); }

// Order-preserving keys of `count` elements.
int oracle_keys(const void* values, int64_t count, int dtype, uint32_t* keys) {
  if (!elem_size(dtype)) return -2;
  const unsigned char* base = static_cast<const unsigned char*>(values);
  for (int64_t i = 0; i < count; ++i) keys[i] = key_at(base, i, dtype);
  return 0;
}

// Exact top-k of each of `rows` contiguous rows of length n.
// out_values: [rows, k] elements of the input dtype (the input's own bits);
// out_indices: [rows, k] row-local int64 indices.  Returns 0, or a negative
// number for bad arguments.
int oracle_topk(const void* values, int64_t n, int64_t rows, int64_t k, int dtype,
                void* out_values, int64_t* out_indices) {
  const int es = elem_size(dtype);
  if (!es) return -2;
  if (n < 1 || rows < 1 || k < 1 || k > n) return -1;
  const unsigned char* base = static_cast<const unsigned char*>(values);
  unsigned char* ov = static_cast<unsigned char*>(out_values);
  std::vector<uint32_t> keys(n);
  std::vector<uint32_t> order(n);
  for (int64_t r = 0; r < rows; ++r) {
    const unsigned char* row = base + r * n * es;
    for (int64_t i = 0; i < n; ++i) {
      keys[i] = key_at(row, i, dtype);
      order[i] = static_cast<uint32_t>(i);
    }
    auto outranks = [&](uint32_t a, uint32_t b) {
      return keys[a] > keys[b] || (keys[a] == keys[b] && a < b);
    };
    std::partial_sort(order.begin(), order.begin() + k, order.end(), outranks);
    for (int64_t j = 0; j < k; ++j) {
      std::memcpy(ov + (r * k + j) * es, row + static_cast<int64_t>(order[j]) * es, es);
      out_indices[r * k + j] = order[j];
    }
  }
  return 0;
}

// The same selection on T threads, for timing the CPU side: each thread
// takes a contiguous chunk of the row and keeps its own first min(k, chunk)
// in rank order; then the union of those lists is partially sorted again.
// Exact, because the k best of a row lie among the k best of whichever chunk
// holds each of them.
int oracle_topk_chunked(const void* values, int64_t n, int64_t rows, int64_t k, int dtype,
                        int threads, void* out_values, int64_t* out_indices) {
  const int es = elem_size(dtype);
  if (!es) return -2;
  if (n < 1 || rows < 1 || k < 1 || k > n || threads < 1) return -1;
  const unsigned char* base = static_cast<const unsigned char*>(values);
  unsigned char* ov = static_cast<unsigned char*>(out_values);
  std::vector<uint32_t> keys(n);
  const int64_t T = threads;
  const int64_t chunk = (n + T - 1) / T;
  std::vector<std::vector<uint32_t>> best(T);
  for (int64_t r = 0; r < rows; ++r) {
    const unsigned char* row = base + r * n * es;
    auto outranks = [&](uint32_t a, uint32_t b) {
      return keys[a] > keys[b] || (keys[a] == keys[b] && a < b);
    };
    std::vector<std::thread> pool;
    for (int64_t c = 0; c < T; ++c) {
      pool.emplace_back([&, c]() {
        const int64_t lo = c * chunk, hi = std::min(n, lo + chunk);
        std::vector<uint32_t>& mine = best[c];
        mine.clear();
        for (int64_t i = lo; i < hi; ++i) {
          keys[i] = key_at(row, i, dtype);
          mine.push_back(static_cast<uint32_t>(i));
        }
        const int64_t keep = std::min<int64_t>(k, static_cast<int64_t>(mine.size()));
        std::partial_sort(mine.begin(), mine.begin() + keep, mine.end(), outranks);
        mine.resize(keep);
      });
    }
    for (auto& th : pool) th.join();
    std::vector<uint32_t> all;
    for (auto& b : best) all.insert(all.end(), b.begin(), b.end());
    std::partial_sort(all.begin(), all.begin() + k, all.end(), outranks);
    for (int64_t j = 0; j < k; ++j) {
      std::memcpy(ov + (r * k + j) * es, row + static_cast<int64_t>(all[j]) * es, es);
      out_indices[r * k + j] = all[j];
    }
  }
  return 0;
}

// First S images of the keyed permutation of [0, n) for (seed, row).
int oracle_sample_indices(uint64_t seed, uint64_t row, uint64_t n, uint64_t S, uint64_t* out) {
  if (S > n || n == 0) return -1;
  Perm p = make_perm(seed, row, n);
  for (uint64_t i = 0; i < S; ++i) out[i] = perm_index(p, i);
  return 0;
}

// Full permutation image of every i in [0, count) (count <= domain size); used
// by the tests to check the Feistel network is a bijection on its domain.
int oracle_feistel_raw(uint64_t seed, uint64_t row, uint64_t n, uint64_t count, uint64_t* out) {
  Perm p = make_perm(seed, row, n);
  uint64_t dom = 1ull << (2 * p.h);
  if (count > dom) return -1;
  for (uint64_t i = 0; i < count; ++i) out[i] = feistel(p, i);
  return 0;
}

// Sample-based threshold of one row: tau = t-th largest key among the S
// sampled elements, R = #{i : key_i >= tau}.  sample_keys (optional, S
// entries) receives the sampled keys in sample order.
int oracle_tau(const void* row_values, uint64_t n, int dtype, uint64_t seed, uint64_t row,
               uint64_t S, uint64_t t, uint32_t* tau_key, uint64_t* R, uint32_t* sample_keys) {
  if (!elem_size(dtype)) return -2;
  if (S < 1 || S > n || t < 1 || t > S) return -1;
  const unsigned char* base = static_cast<const unsigned char*>(row_values);
  Perm p = make_perm(seed, row, n);
  std::vector<uint32_t> sk(S);
  for (uint64_t i = 0; i < S; ++i) sk[i] = key_at(base, static_cast<int64_t>(perm_index(p, i)), dtype);
  if (sample_keys) std::memcpy(sample_keys, sk.data(), S * 4);
  std::vector<uint32_t> sorted = sk;
  std::sort(sorted.begin(), sorted.end(), [](uint32_t a, uint32_t b) { return a > b; });
  uint32_t tau = sorted[t - 1];
  uint64_t cnt = 0;
  for (uint64_t i = 0; i < n; ++i) cnt += key_at(base, static_cast<int64_t>(i), dtype) >= tau;
  *tau_key = tau;
  *R = cnt;
  return 0;
}

}  // extern "C"
