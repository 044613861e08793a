// Large k: tile sort and merges (buffers above the bucket sort), the dispatch macro, and the bucket sort kernels.
// A part of topk_kernels.hip, included there in order inside namespace tk;
// it relies on the definitions of the parts before it and is not a
// stand-alone header.
#pragma once

// ======================================================================
// Large k: sort all candidates by composite (descending) and keep the first
// k.  Tiles of SORT_TILE are bitonic-sorted in LDS, then runs are merged
// pairwise; each element finds its place in the merged run from its own
// position plus a binary search for the number of larger elements in the
// partner run (the lower-bound search of GPU.js Learn "Find It in log n";
// composites are unique, so there are no ties to break).
// ======================================================================
constexpr uint32_t SORT_TILE = 4096;

__global__ __launch_bounds__(SEL_THREADS) void k_tile_sort(RowState* __restrict__ states,
                                                           uint64_t* __restrict__ cbuf,
                                                           uint32_t cap) {
  __shared__ uint64_t x[SORT_TILE];
  const uint32_t row = blockIdx.y, tid = threadIdx.x;
  const uint32_t R = min(states[row].count, cap);
  const uint32_t start = blockIdx.x * SORT_TILE;
  if (start >= R) return;
  const uint32_t len = min(SORT_TILE, R - start);
  uint64_t* p = cbuf + (size_t)row * cap + start;
  uint64_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t i = 4 * tid + (uint32_t)j;
    v[j] = i < len ? p[i] : 0ull;   // composites are never 0: padding sorts last
  }
  block_bitonic4096_desc(v, x);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t i = 4 * tid + (uint32_t)j;
    if (i < len) p[i] = v[j];
  }
}

__global__ __launch_bounds__(256) void k_merge(RowState* __restrict__ states,
                                               const uint64_t* __restrict__ src,
                                               uint64_t* __restrict__ dst, uint32_t cap,
                                               uint32_t run) {
  const uint32_t row = blockIdx.y;
  const uint32_t R = min(states[row].count, cap);
  const uint32_t p = blockIdx.x * 256u + threadIdx.x;
  if (p >= R) return;
  const uint64_t* a = src + (size_t)row * cap;
  uint64_t* d = dst + (size_t)row * cap;
  const uint32_t r = p / run;
  const uint32_t pair_lo = (r & ~1u) * run;
  const uint32_t mid = min(pair_lo + run, R);
  const uint32_t end = min(pair_lo + 2 * run, R);
  const uint64_t x = a[p];
  uint32_t o, lo, hi;
  if ((r & 1u) == 0) {  // left run: count larger elements of the right run
    o = p - pair_lo;
    lo = mid;
    hi = end;
  } else {
    o = p - mid;
    lo = pair_lo;
    hi = mid;
  }
  const uint32_t base = lo;
  while (lo < hi) {
    const uint32_t m = (lo + hi) >> 1;
    if (a[m] > x) lo = m + 1;
    else hi = m;
  }
  d[pair_lo + o + (lo - base)] = x;
}

template <int DT>
__global__ __launch_bounds__(256) void k_output(const void* __restrict__ values, uint32_t n,
                                                RowState* __restrict__ states,
                                                const uint64_t* __restrict__ sorted, uint32_t cap,
                                                uint32_t k, uint32_t B, void* __restrict__ out_values,
                                                int64_t* __restrict__ out_idx) {
  const uint32_t row = blockIdx.y;
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= k) return;
  if (i >= min(states[row].count, cap)) {   // a row that keeps fewer than k
    store_pad<DT>(out_values, out_idx, (size_t)row * k + i);
    return;
  }
  const uint64_t c = sorted[(size_t)row * cap + i];
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
  uint32_t idx;
  const uint32_t bits = winner_bits<DT>(c, B, rowp, n, &idx);
  store_winner<DT>(out_values, out_idx, (size_t)row * k + i, bits, idx);
  if (i == 0) states[row].status = ST_DONE;
}

// ======================================================================
// Launchers
// ======================================================================
#define TK_DISPATCH(dt, KERNEL, ...)                                          \
  switch (dt) {                                                               \
    case DT_I32: hipLaunchKernelGGL(KERNEL<DT_I32>, __VA_ARGS__); break;      \
    case DT_F32: hipLaunchKernelGGL(KERNEL<DT_F32>, __VA_ARGS__); break;      \
    default: hipLaunchKernelGGL(KERNEL<DT_BF16>, __VA_ARGS__); break;         \
  }

__global__ __launch_bounds__(LK_THREADS) void k_lk_hist(const RowState* __restrict__ states,
                                                        const uint64_t* __restrict__ cbuf,
                                                        uint32_t cap, uint32_t B, uint32_t bl,
                                                        uint32_t* __restrict__ lk) {
  __shared__ uint32_t h[LK_BINS];
  const uint32_t row = blockIdx.y, tid = threadIdx.x;
  const RowState st = states[row];
  const uint32_t R = st.count < cap ? st.count : cap;
  const uint32_t base = blockIdx.x * LK_CHUNK;
  if (st.status != ST_SORT || base >= R) return;
  const LkDigit g = lk_digit_of(st, B, bl);
  for (uint32_t i = tid; i < LK_BINS; i += LK_THREADS) h[i] = 0;
  __syncthreads();
  const uint64_t* p = cbuf + (size_t)row * cap;
  uint64_t c[4];
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t i = base + j * LK_THREADS + tid;
    c[j] = i < R ? p[i] : 0ull;
  }
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j)
    if (base + j * LK_THREADS + tid < R) atomicAdd(&h[g(c[j])], 1u);
  __syncthreads();
  uint32_t* gh = lk + (size_t)row * LK_BINS;
  for (uint32_t i = tid; i < LK_BINS; i += LK_THREADS)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(LK_THREADS) void k_lk_scatter(const RowState* __restrict__ states,
                                                           const uint64_t* __restrict__ cbuf,
                                                           uint64_t* __restrict__ aux, uint32_t cap,
                                                           uint32_t k, uint32_t B, uint32_t bl,
                                                           uint32_t* __restrict__ lk,
                                                           uint32_t rows) {
  __shared__ uint32_t s_start[LK_BINS];   // by rank
  __shared__ uint32_t s_cnt[LK_BINS];     // this workgroup's count, then its base, per rank
  __shared__ uint32_t s_wsum[LK_THREADS / 64];
  __shared__ uint32_t s_win[2 * LK_MAXWIN];
  const uint32_t row = blockIdx.y, tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
  const RowState st = states[row];
  const uint32_t R = st.count < cap ? st.count : cap;
  const uint32_t base = blockIdx.x * LK_CHUNK;
  if (st.status != ST_SORT || base >= R) return;
  const LkDigit g = lk_digit_of(st, B, bl);
  const uint32_t* gh = lk + (size_t)row * LK_BINS;
  uint32_t* gfill = lk + (size_t)(rows + row) * LK_BINS;
  uint32_t* gstart = lk + (size_t)2 * rows * LK_BINS + (size_t)row * LK_STRIDE;
  // this workgroup's candidates, loaded first so the histogram read overlaps
  const uint64_t* p = cbuf + (size_t)row * cap;
  uint64_t c[4];
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t i = base + j * LK_THREADS + tid;
    c[j] = i < R ? p[i] : 0ull;
  }

  // bucket starts in descending bucket order: thread t owns ranks 4t..4t+3
  uint32_t hv[4], sum = 0;
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    hv[j] = gh[LK_BINS - 1 - (4 * tid + j)];
    sum += hv[j];
  }
  const uint32_t incl = wave_incl_sum(sum);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  uint32_t run = incl - sum;
#pragma unroll
  for (uint32_t i = 0; i < LK_THREADS / 64; ++i) run += i < w ? s_wsum[i] : 0u;
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    s_start[4 * tid + j] = run;
    s_cnt[4 * tid + j] = 0;
    if (blockIdx.x == 0) gstart[4 * tid + j] = run;
    run += hv[j];
  }
  if (blockIdx.x == 0 && tid == LK_THREADS - 1) gstart[LK_BINS] = run;
  if (blockIdx.x == 0)
    for (uint32_t i = tid; i < 2 * LK_MAXWIN; i += LK_THREADS) s_win[i] = i < LK_MAXWIN ? ~0u : 0u;
  __syncthreads();
  if (blockIdx.x == 0) {
    // each sort window: first and last non-empty bucket starting in it
    const uint32_t nwin = (k + LK_WIN - 1) / LK_WIN;
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
      const uint32_t rr = 4 * tid + j, b0 = s_start[rr];
      if (hv[j] && b0 < k) {
        atomicMin(&s_win[b0 / LK_WIN], rr);
        atomicMax(&s_win[LK_MAXWIN + b0 / LK_WIN], rr);
      }
    }
    __syncthreads();
    uint32_t* gwin = lk + (size_t)rows * (2 * LK_BINS + LK_STRIDE) + (size_t)row * 2 * LK_MAXWIN;
    for (uint32_t i = tid; i < nwin; i += LK_THREADS) {
      gwin[i] = s_win[i];
      gwin[LK_MAXWIN + i] = s_win[LK_MAXWIN + i];
    }
  }

  // this workgroup's candidates: local rank inside its bucket
  uint32_t r[4], lr[4];
  bool need[4];
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t i = base + j * LK_THREADS + tid;
    const bool ok = i < R;
    r[j] = ok ? LK_BINS - 1 - g(c[j]) : 0u;
    need[j] = ok && s_start[r[j]] < k;
    lr[j] = need[j] ? atomicAdd(&s_cnt[r[j]], 1u) : 0u;
  }
  __syncthreads();
  // one reservation per bucket and workgroup
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t rr = 4 * tid + j;
    const uint32_t cnt = s_cnt[rr];
    if (cnt) s_cnt[rr] = atomicAdd(&gfill[rr], cnt);
  }
  __syncthreads();
  uint64_t* a = aux + (size_t)row * cap;   // compacted values, by bucket
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j)
    if (need[j]) a[s_start[r[j]] + s_cnt[r[j]] + lr[j]] = g.compact(c[j]);
}

template <int DT>
__global__ __launch_bounds__(LK_THREADS) void k_lk_sort(
    const void* __restrict__ values, uint32_t n, const RowState* __restrict__ states,
    CallState* __restrict__ cs, uint64_t* __restrict__ aux, uint64_t* __restrict__ scratch,
    uint32_t cap, uint32_t k, uint32_t B, uint32_t bl, uint32_t* __restrict__ lk, uint32_t rows,
    void* __restrict__ out_values, int64_t* __restrict__ out_idx) {
  __shared__ uint64_t s_a[LK_LCAP];
  __shared__ uint64_t s_b[LK_LCAP];
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_runs[2 * 2048];
  __shared__ uint32_t s_frames[3 * LK_STACK];
  __shared__ uint64_t s_red[32];
  __shared__ uint32_t s_misc[8];
  __shared__ uint32_t s_sm[8];
  const uint32_t row = blockIdx.y, tid = threadIdx.x, nt = LK_THREADS;
  const uint32_t lane = tid & 63u, w = tid >> 6;
  const RowState st = states[row];
  if (st.status != ST_SORT) return;
  const uint32_t R = st.count < cap ? st.count : cap;
  if (R < k) {   // a row that keeps fewer than k: pad this window's slots past R
    const uint32_t w0 = blockIdx.x * LK_WIN, w1 = w0 + LK_WIN < k ? w0 + LK_WIN : k;
    for (uint32_t i = (w0 > R ? w0 : R) + tid; i < w1; i += nt)
      store_pad<DT>(out_values, out_idx, (size_t)row * k + i);
  }
  const uint32_t* gs = lk + (size_t)2 * rows * LK_BINS + (size_t)row * LK_STRIDE;
  const uint32_t* gwin = lk + (size_t)rows * (2 * LK_BINS + LK_STRIDE) + (size_t)row * 2 * LK_MAXWIN;
  if (blockIdx.x * LK_WIN >= k) return;
  // the non-empty buckets that start in this window and below k
  const uint32_t r_lo = gwin[blockIdx.x];
  if (r_lo == ~0u) return;
  const uint32_t r_end = gwin[LK_MAXWIN + blockIdx.x] + 1;

  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
  uint64_t* A = aux + (size_t)row * cap;
  uint64_t* S = scratch + (size_t)row * cap;
  const LkDigit g = lk_digit_of(st, B, bl);

  // sort [lo, lo + len) of src (compacted values, unique, len <= LK_LCAP) in
  // LDS and write the output positions below k.  nb > 0: the range is the
  // buckets of ranks r_last - nb + 1 .. r_last, and the sort's bins are the
  // bucket and the bits just below the bucket digit; nb = 0: bins from the
  // range's extremes.
  auto sort_out = [&](const uint64_t* src, uint32_t lo, uint32_t len, uint32_t nb,
                      uint32_t r_last) {
    for (uint32_t i = tid; i < len; i += nt) s_a[i] = src[lo + i];
    __syncthreads();
    bool ok;
    if (nb > 0 && nb <= 2048) {
      uint32_t sb = 31u - (uint32_t)__builtin_clz(2048u / nb);   // nb << sb <= 2048
      if (sb > g.shift) sb = g.shift;
      const uint32_t dsh = g.shift - sb;
      const uint64_t dbase = (uint64_t)(LK_BINS - 1 - r_last) << sb;
      ok = block_sort_binned_desc(s_a, len, s_b, s_hist, s_sm, reinterpret_cast<uint32_t*>(s_red),
                                  [&](uint64_t v) { return (uint32_t)((v >> dsh) - dbase); }, 64u);
    } else {
      ok = block_sort_unique_desc(s_a, len, s_b, s_hist, s_sm, s_red, 64u);
    }
    if (!ok) {
      // crowded top bits: bitonic sort instead (zero padding sorts last; a
      // value of 0 is the range's smallest, so it still lands in place)
      const uint32_t P = next_pow2(len);
      for (uint32_t i = len + tid; i < P; i += nt) s_a[i] = 0ull;
      __syncthreads();
      block_bitonic_desc(s_a, P);
    }
    for (uint32_t i = tid; i < len; i += nt) {
      const uint32_t pos = lo + i;
      if (pos < k) {
        uint32_t idx;
        const uint32_t bits = winner_bits<DT>(g.expand(s_a[i]), B, rowp, n, &idx);
        store_winner<DT>(out_values, out_idx, (size_t)row * k + pos, bits, idx);
      }
    }
    __syncthreads();
  };

  // oversized ranges, split further (frames: lo, len, 1 = data in S)
  uint32_t sp = 0;   // uniform
  auto push = [&](uint32_t lo, uint32_t len, uint32_t in_s) {
    if (sp < LK_STACK) {
      if (tid == 0) {
        s_frames[3 * sp] = lo;
        s_frames[3 * sp + 1] = len;
        s_frames[3 * sp + 2] = in_s;
      }
      ++sp;
    } else if (tid == 0) {
      atomicOr(&cs->error, 2u);   // cannot happen: see LK_STACK
    }
  };

  const uint32_t a0 = gs[r_lo], e0 = gs[r_end], last = gs[r_end - 1];
  if (e0 - a0 <= LK_LCAP) {
    sort_out(A, a0, e0 - a0, r_end - r_lo, r_end - 1);
  } else {
    // every bucket but the last starts and ends inside the window
    if (last > a0) sort_out(A, a0, last - a0, r_end - 1 - r_lo, r_end - 2);
    if (e0 - last <= LK_LCAP) sort_out(A, last, e0 - last, 1u, r_end - 1);
    else push(last, e0 - last, 0u);
  }
  __syncthreads();

  while (sp > 0) {
    --sp;
    const uint32_t lo = s_frames[3 * sp], len = s_frames[3 * sp + 1];
    const bool in_s = s_frames[3 * sp + 2] != 0;
    __syncthreads();
    const uint64_t* src = in_s ? S : A;
    uint64_t* dst = in_s ? A : S;
    // 11-bit digit just below the common prefix of the range's extremes
    uint64_t mn = ~0ull, mx = 0ull;
    for (uint32_t i = tid; i < len; i += nt) {
      const uint64_t v = src[lo + i];
      mn = v < mn ? v : mn;
      mx = v > mx ? v : mx;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const uint64_t x = __shfl_xor(mn, d, 64), y = __shfl_xor(mx, d, 64);
      mn = x < mn ? x : mn;
      mx = y > mx ? y : mx;
    }
    if (lane == 0) {
      s_red[w] = mn;
      s_red[16 + w] = mx;
    }
    for (uint32_t i = tid; i < 2048; i += nt) s_hist[i] = 0;
    __syncthreads();
    mn = s_red[0];
    mx = s_red[16];
    for (uint32_t j = 1; j < nt / 64; ++j) {
      mn = s_red[j] < mn ? s_red[j] : mn;
      mx = s_red[16 + j] > mx ? s_red[16 + j] : mx;
    }
    const uint32_t top = 63u - (uint32_t)__builtin_clzll(mn ^ mx);   // len >= 2: unique values differ
    const uint32_t sh = top >= 10 ? top - 10 : 0u;
    auto digit = [&](uint64_t v) { return (uint32_t)(v >> sh) & 2047u; };
    for (uint32_t i = tid; i < len; i += nt) atomicAdd(&s_hist[digit(src[lo + i])], 1u);
    __syncthreads();
    if (w == 0) {   // exclusive scan from digit 2047 down; lane owns 32 digits
      uint32_t loc = 0;
      for (uint32_t j = 0; j < 32; ++j) loc += s_hist[2047 - (lane * 32 + j)];
      const uint32_t inc = wave_incl_sum(loc);
      uint32_t run = inc - loc;
      for (uint32_t j = 0; j < 32; ++j) {
        const uint32_t b = 2047 - (lane * 32 + j);
        const uint32_t h = s_hist[b];
        s_hist[b] = run;
        run += h;
      }
    }
    __syncthreads();
    for (uint32_t i = tid; i < len; i += nt) {
      const uint64_t v = src[lo + i];
      dst[lo + atomicAdd(&s_hist[digit(v)], 1u)] = v;
    }
    __syncthreads();
    // s_hist[b] is now the end of digit b's range; pack consecutive digits
    // into runs of at most LK_LCAP (one thread; this path is rare)
    if (tid == 0) {
      uint32_t nr = 0, cur = 0, cl = 0;
      for (int b = 2047; b >= 0; --b) {
        const uint32_t beg = (b == 2047) ? 0u : s_hist[b + 1];
        const uint32_t end = s_hist[b];
        if (end == beg) continue;
        if (lo + beg >= k) break;
        const uint32_t h = end - beg;
        if (h > LK_LCAP) {
          if (cl) {
            s_runs[2 * nr] = cur;
            s_runs[2 * nr + 1] = cl;
            ++nr;
            cl = 0;
          }
          s_runs[2 * nr] = beg;
          s_runs[2 * nr + 1] = h | 0x80000000u;
          ++nr;
          continue;
        }
        if (cl + h > LK_LCAP) {
          s_runs[2 * nr] = cur;
          s_runs[2 * nr + 1] = cl;
          ++nr;
          cl = 0;
        }
        if (cl == 0) cur = beg;
        cl += h;
      }
      if (cl) {
        s_runs[2 * nr] = cur;
        s_runs[2 * nr + 1] = cl;
        ++nr;
      }
      s_misc[2] = nr;
    }
    __syncthreads();
    const uint32_t nr = s_misc[2];
    for (uint32_t q = 0; q < nr; ++q) {
      const uint32_t rs = s_runs[2 * q], rl = s_runs[2 * q + 1];
      if (rl & 0x80000000u) push(lo + rs, rl & 0x7FFFFFFFu, in_s ? 0u : 1u);
      else sort_out(dst, lo + rs, rl, 0u, 0u);
      __syncthreads();
    }
  }
}
