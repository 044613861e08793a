// Workgroup-level radix select on composites (one workgroup per row).
//
// Radix selection counts elements into digit buckets and recurses into the
// bucket that holds the boundary (GPU.js Learn "Find the Cutoff Instead",
// section "Same idea elsewhere").  Here the digits are 8 bits of the
// composite, taken from the top, the histograms live in LDS, and once the
// boundary bucket is small enough its elements are copied into LDS so the
// remaining passes never touch global memory.
#pragma once

#include "topk_device.hpp"

namespace tk {

// Add one element (digit `d`, if `active`) to an LDS histogram.  All 64 lanes
// of the wave must call it together.  When every active lane has the same
// digit, one lane adds the whole count (skewed data hits one bin).
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t d, bool active) {
  uint64_t act = ballot(active);
  if (!act) return;
  const uint32_t first = (uint32_t)__builtin_ctzll(act);
  const uint32_t d0 = wave_bcast(d, first);
  const uint64_t same = ballot(active && d == d0);
  if (same == act) {
    if (lane_id() == first) atomicAdd(&h[d0], (uint32_t)__builtin_popcountll(act));
  } else if (active) {
    atomicAdd(&h[d], 1u);
  }
}

// Append `c` (if `keep`) to an LDS array through a shared counter; all lanes
// of the wave call it together.
// Slots at or beyond `cap` are counted but not written.
__device__ __forceinline__ void lds_append(uint64_t* arr, uint32_t* counter, uint32_t cap,
                                           uint64_t c, bool keep) {
  uint64_t m = ballot(keep);
  if (!m) return;
  uint32_t base = 0;
  const uint32_t first = (uint32_t)__builtin_ctzll(m);
  if (lane_id() == first) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = wave_bcast(base, first);
  const uint32_t slot = base + rank_below(m);
  if (keep && slot < cap) arr[slot] = c;
}

// Loop over i in [0, total) with U loads in flight per thread: `load(i)` for
// every valid i first, then `proc(value, valid)` in order.  Every thread of
// the workgroup runs the same trip count, so proc may use wave operations.
template <int U, class T, class Load, class Proc>
__device__ __forceinline__ void for_batched(uint32_t total, Load&& load, Proc&& proc) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  for (uint32_t i0 = 0; i0 < total; i0 += nt * U) {
    T v[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = i0 + (uint32_t)u * nt + tid;
      ok[u] = i < total;
      v[u] = ok[u] ? load(i) : T(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) proc(v[u], ok[u]);
  }
}

// Same, with the element index passed to proc(value, valid, i).
template <int U, class T, class Load, class Proc>
__device__ __forceinline__ void for_batched_i(uint32_t total, Load&& load, Proc&& proc) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  for (uint32_t i0 = 0; i0 < total; i0 += nt * U) {
    T v[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = i0 + (uint32_t)u * nt + tid;
      ok[u] = i < total;
      v[u] = ok[u] ? load(i) : T(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) proc(v[u], ok[u], i0 + (uint32_t)u * nt + tid);
  }
}

constexpr int LOADS_IN_FLIGHT = 8;

// Append a 32-bit value to an LDS list (same rules as lds_append).
__device__ __forceinline__ void lds_append_u32(uint32_t* arr, uint32_t* counter, uint32_t cap,
                                               uint32_t v, bool keep) {
  uint64_t m = ballot(keep);
  if (!m) return;
  uint32_t base = 0;
  const uint32_t first = (uint32_t)__builtin_ctzll(m);
  if (lane_id() == first) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = wave_bcast(base, first);
  const uint32_t slot = base + rank_below(m);
  if (keep && slot < cap) arr[slot] = v;
}

struct SelectOut {
  uint64_t thr;       // threshold composite: resolved top bits, zeros below
  uint32_t count_ge;  // elements with composite >= thr
};

// Where a select starts: `nb` top bits already resolved to `prefix` (bits
// below zero), `above` elements known to lie above that prefix, and the rank
// `need` still wanted inside it.  With in_lds, the `m` elements matching the
// prefix already sit in s_cand.
struct SelectStart {
  uint64_t prefix = 0;
  uint32_t nb = 0, need = 1, above = 0, m = 0;
  bool in_lds = false;
};

// Select over `n` composites produced by `src(i)` (W significant bits): the
// composite of rank `need` (1-based, from the top) among those matching the
// start prefix.  Digits are 8 bits from the top (the last may be narrower).
// Passes stop as soon as the elements >= the bucket's lower edge number at
// most `stop` (pass stop = 0 to resolve every bit).
//
// LDS: s_hist[256], s_misc[8], s_cand[cand_cap].  Every thread of the
// workgroup must call it.
template <class Src>
__device__ SelectOut block_select_from(const Src& src, uint32_t n, uint32_t W, SelectStart st0,
                                       uint32_t stop, uint32_t* s_hist, uint32_t* s_misc,
                                       uint64_t* s_cand, uint32_t cand_cap) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  uint64_t prefix = st0.prefix;
  uint32_t nb = st0.nb, need = st0.need, above = st0.above, m = st0.m;
  bool in_lds = st0.in_lds;
  for (;;) {
    const uint32_t width = (W - nb) < 8u ? (W - nb) : 8u;
    const uint32_t shift = W - nb - width;
    const uint32_t pshift = W - nb;            // bits below the resolved prefix
    const uint64_t ptop = nb ? (prefix >> pshift) : 0;
    const uint32_t dmask = (1u << width) - 1u;
    for (uint32_t i = tid; i < 256; i += nt) s_hist[i] = 0;
    __syncthreads();
    auto count = [&](uint64_t c, bool ok) {
      const bool act = ok && ((nb == 0) || ((c >> pshift) == ptop));
      hist_add(s_hist, (uint32_t)(c >> shift) & dmask, act);
    };
    if (in_lds) {
      for (uint32_t i0 = 0; i0 < m; i0 += nt) {
        const uint32_t i = i0 + tid;
        count(i < m ? s_cand[i] : 0ull, i < m);
      }
    } else {
      for_batched<LOADS_IN_FLIGHT, uint64_t>(n, [&](uint32_t i) { return src(i); }, count);
    }
    __syncthreads();
    if (tid < 64) wave_find_bucket(s_hist, need, s_misc);
    __syncthreads();
    const uint32_t b = s_misc[0], acc = s_misc[1], hb = s_misc[2];
    above += acc;
    need -= acc;
    prefix |= (uint64_t)b << shift;
    nb += width;
    const uint32_t count_ge = above + hb;
    if (count_ge <= stop || nb >= W) {
      __syncthreads();
      return SelectOut{prefix, count_ge};
    }
    if (!in_lds && hb <= cand_cap) {
      // copy the boundary bucket into LDS
      const uint32_t npshift = W - nb;
      const uint64_t ntop = prefix >> npshift;
      if (tid == 0) s_misc[3] = 0;
      __syncthreads();
      for_batched<LOADS_IN_FLIGHT, uint64_t>(
          n, [&](uint32_t i) { return src(i); },
          [&](uint64_t c, bool ok) {
            lds_append(s_cand, &s_misc[3], cand_cap, c, ok && (c >> npshift) == ntop);
          });
      __syncthreads();
      m = s_misc[3] < cand_cap ? s_misc[3] : cand_cap;
      in_lds = true;
    }
    __syncthreads();
  }
}

template <class Src>
__device__ SelectOut block_select(const Src& src, uint32_t n, uint32_t W, uint32_t rank,
                                  uint32_t stop, uint32_t* s_hist, uint32_t* s_misc,
                                  uint64_t* s_cand, uint32_t cand_cap) {
  SelectStart st;
  st.need = rank;
  return block_select_from(src, n, W, st, stop, s_hist, s_misc, s_cand, cand_cap);
}

// Over an LDS histogram of `nbins` bins (a power of two, at most 4096) taken
// from the top, find the bin b holding rank `need` (1-based): out[0] = b,
// out[1] = elements in bins above b, out[2] = hist[b].  Needs need <= total.
// Every thread of the workgroup calls it; s_tmp holds 16 words.
__device__ __forceinline__ void block_find_bucket(const uint32_t* hist, uint32_t nbins,
                                                  uint32_t need, uint32_t* out, uint32_t* s_tmp) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  const uint32_t per = nbins > nt ? nbins / nt : 1u;   // bins per thread
  const uint32_t used = nbins / per;                   // threads holding bins
  const uint32_t lane = tid & 63u, w = tid >> 6;
  uint32_t s = 0;
  if (tid < used) {
    for (uint32_t j = 0; j < per; ++j) s += hist[nbins - 1 - (tid * per + j)];
  }
  uint32_t incl = wave_incl_sum(s);
  if (lane == 63) s_tmp[w] = incl;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (uint32_t j = 0; j < 16; ++j) base += j < w ? s_tmp[j] : 0u;   // independent reads
  incl += base;
  const uint32_t excl = incl - s;
  if (tid < used && excl < need && need <= incl) {
    uint32_t acc = excl;
    for (uint32_t j = 0; j < per; ++j) {
      const uint32_t b = nbins - 1 - (tid * per + j);
      const uint32_t h = hist[b];
      if (acc + h >= need) {
        out[0] = b;
        out[1] = acc;
        out[2] = h;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// Gather every composite >= thr from `src` into s_out (LDS) in any order;
// returns how many.  Every thread must call it.
template <class Src>
__device__ uint32_t block_collect(const Src& src, uint32_t n, uint64_t thr, uint64_t* s_out,
                                  uint32_t out_cap, uint32_t* s_counter) {
  const uint32_t tid = threadIdx.x;
  if (tid == 0) *s_counter = 0;
  __syncthreads();
  for_batched<LOADS_IN_FLIGHT, uint64_t>(
      n, [&](uint32_t i) { return src(i); },
      [&](uint64_t c, bool ok) { lds_append(s_out, s_counter, out_cap, c, ok && c >= thr); });
  __syncthreads();
  const uint32_t cnt = *s_counter;
  __syncthreads();
  return cnt < out_cap ? cnt : out_cap;
}

// Bitonic sort of s[0..P) into descending order, P a power of two.
__device__ __forceinline__ void block_bitonic_desc(uint64_t* s, uint32_t P) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t i = tid; i < (P >> 1); i += nt) {
        const uint32_t lo = (i / stride) * (stride << 1) + (i % stride);
        const uint32_t hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = s[lo], c = s[hi];
        if (desc ? (a < c) : (a > c)) {
          s[lo] = c;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- LDS sort
// Exclusive scan of hist[0..2048) from bin 2047 down: on return hist[b] is
// the number of elements in the bins above b.  wsum: 16 words of scratch.
// Every thread of the workgroup calls it.
__device__ __forceinline__ void block_scan_desc_2048(uint32_t* hist, uint32_t* wsum) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x, lane = tid & 63u, w = tid >> 6;
  const uint32_t per = 2048u / nt;   // bins per thread, in descending order
  uint32_t loc = 0;
  for (uint32_t j = 0; j < per; ++j) loc += hist[2047u - (tid * per + j)];
  const uint32_t incl = wave_incl_sum(loc);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t run = incl - loc;
#pragma unroll
  for (uint32_t i = 0; i < 16; ++i) run += i < w ? wsum[i] : 0u;
  for (uint32_t j = 0; j < per; ++j) {
    const uint32_t b = 2047u - (tid * per + j);
    const uint32_t h = hist[b];
    hist[b] = run;
    run += h;
  }
  __syncthreads();
}

// Sort cnt unique 64-bit values s[0..cnt) into descending order, in LDS,
// given digit(v) in [0, 2048) that never decreases as v grows: a counting
// sort on the digit, then each element's place inside its bin is the number
// of larger values in that bin.  O(cnt) LDS passes plus the sum of squared
// bin sizes.  tmp: cnt values of scratch; hist: 2048 words; misc: 8 words;
// wsum: 16 words.  Every thread of the workgroup calls it.  Returns false,
// with s untouched, when the fullest bin holds more than max_bin values; the
// caller then sorts another way.
template <class Digit>
__device__ __forceinline__ bool block_sort_binned_desc(uint64_t* s, uint32_t cnt, uint64_t* tmp,
                                                       uint32_t* hist, uint32_t* misc,
                                                       uint32_t* wsum, Digit&& digit,
                                                       uint32_t max_bin) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  for (uint32_t i = tid; i < 2048; i += nt) hist[i] = 0;
  if (tid == 0) misc[0] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < cnt; i += nt) atomicAdd(&hist[digit(s[i])], 1u);
  __syncthreads();
  {
    uint32_t big = 0;
    for (uint32_t i = tid; i < 2048; i += nt) big = hist[i] > big ? hist[i] : big;
    if (big > max_bin) atomicMax(&misc[0], big);
  }
  __syncthreads();
  if (misc[0] > max_bin) {
    __syncthreads();
    return false;
  }
  block_scan_desc_2048(hist, wsum);   // hist[b] = start of bin b (a cursor below)
  // scatter into bins (order inside a bin arbitrary for now)
  for (uint32_t i = tid; i < cnt; i += nt) {
    const uint64_t v = s[i];
    tmp[atomicAdd(&hist[digit(v)], 1u)] = v;
  }
  __syncthreads();
  // hist[b] is now the end of bin b; its start is the end of the bin above
  // it (b + 1), or 0 for the top bin
  for (uint32_t p = tid; p < cnt; p += nt) {
    const uint64_t v = tmp[p];
    const uint32_t b = digit(v);
    const uint32_t end = hist[b];
    const uint32_t beg = (b == 2047) ? 0u : hist[b + 1];
    uint32_t r = 0;
    for (uint32_t q = beg; q < end; ++q) r += (tmp[q] > v) ? 1u : 0u;
    s[beg + r] = v;
  }
  __syncthreads();
  return true;
}

// The same with the digit taken as the 11 bits just below the common prefix
// of the smallest and largest value (digits from the top, so bin order is
// value order).  red: 32 words of scratch.
__device__ __forceinline__ bool block_sort_unique_desc(uint64_t* s, uint32_t cnt, uint64_t* tmp,
                                                       uint32_t* hist, uint32_t* misc,
                                                       uint64_t* red, uint32_t max_bucket) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x, lane = tid & 63u, w = tid >> 6;
  if (cnt <= 1) {
    __syncthreads();
    return true;
  }
  uint64_t mn = ~0ull, mx = 0ull;
  for (uint32_t i = tid; i < cnt; i += nt) {
    const uint64_t v = s[i];
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
  }
  mn = wave_min_u64(mn);
  mx = wave_max_u64(mx);
  if (lane == 0) {
    red[w] = mn;
    red[16 + w] = mx;
  }
  __syncthreads();
  const uint32_t nw = nt >> 6;
#pragma unroll
  for (uint32_t j = 0; j < 16; ++j) {   // independent reads
    const uint64_t a = j < nw ? red[j] : ~0ull, b = j < nw ? red[16 + j] : 0ull;
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  __syncthreads();   // red is reused as scan scratch below
  const uint64_t diff = mn ^ mx;
  const uint32_t top = 63u - (uint32_t)__builtin_clzll(diff);   // diff != 0: values unique
  const uint32_t shift = top >= 10 ? top - 10 : 0u;
  return block_sort_binned_desc(
      s, cnt, tmp, hist, misc, reinterpret_cast<uint32_t*>(red),
      [&](uint64_t v) { return (uint32_t)(v >> shift) & 2047u; }, max_bucket);
}

// Bitonic sort of 4096 values into descending order by 1024 threads, four
// consecutive positions per thread (position p = 4 * tid + j).  Pairs that
// are in one thread swap in registers, pairs within a wave exchange through
// cross-lane shuffles, and only strides of 256 and more go through LDS
// (x: 4096 words of scratch).  Every thread of the workgroup calls it.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, uint32_t m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void block_bitonic4096_desc(uint64_t (&v)[4], uint64_t* x) {
  const uint32_t tid = threadIdx.x;
  for (uint32_t size = 2; size <= 4096; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 256) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[4 * tid + j] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t p = 4 * tid + (uint32_t)j;
          const uint64_t o = x[p ^ stride];
          const bool desc = (p & size) == 0, low = (p & stride) == 0;
          const uint64_t hi = v[j] > o ? v[j] : o, lo = v[j] > o ? o : v[j];
          v[j] = (low == desc) ? hi : lo;
        }
        __syncthreads();
      } else if (stride >= 4) {
        const uint32_t m = stride >> 2;   // partner lane distance
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t p = 4 * tid + (uint32_t)j;
          const uint64_t o = shfl_xor_u64(v[j], m);
          const bool desc = (p & size) == 0, low = (p & stride) == 0;
          const uint64_t hi = v[j] > o ? v[j] : o, lo = v[j] > o ? o : v[j];
          v[j] = (low == desc) ? hi : lo;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = j ^ (int)stride;
          if (q > j) {
            const uint32_t p = 4 * tid + (uint32_t)j;
            const bool desc = (p & size) == 0;
            const uint64_t a = v[j], b = v[q];
            const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
            v[j] = desc ? hi : lo;
            v[q] = desc ? lo : hi;
          }
        }
      }
    }
  }
}

__host__ __device__ __forceinline__ uint32_t next_pow2(uint32_t v) {
  uint32_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace tk
