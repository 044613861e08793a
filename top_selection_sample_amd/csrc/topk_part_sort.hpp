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

// The chunk step of the bucket sort for rows that never pass through the
// finish kernel (the one-workgroup route's large-k rows): one chunk per
// workgroup.
__global__ __launch_bounds__(LK_THREADS) void k_lk_chunk(const RowState* __restrict__ states,
                                                         uint64_t* __restrict__ cbuf, uint32_t cap,
                                                         uint32_t B, uint32_t bl,
                                                         uint32_t* __restrict__ lkc) {
  __shared__ uint32_t h[LK_BINS + 16];
  __shared__ uint64_t s_sorted[LK_CHUNK];
  const uint32_t row = blockIdx.y;
  const RowState st = states[row];
  const uint32_t R = st.count < cap ? st.count : cap;
  const uint32_t base = blockIdx.x * LK_CHUNK;
  if (st.status != ST_SORT || base >= R) return;
  uint64_t* cb = cbuf + (size_t)row * cap;
  lk_sort_chunk(cb, cb, R, R, base, lk_digit_of(st, B, bl), cb,
                lkc + ((size_t)row * lk_maxch(cap) + blockIdx.x) * LK_CSTRIDE, h, s_sorted);
}

// One workgroup per LK_WIN output positions of a row.  cbuf: the row's
// candidates grouped by rank within each chunk (the chunk step), lkc their
// prefix counts; aux: the window's candidates gathered by bucket, as v
// values; scratch: the split's second buffer.
template <int DT>
__global__ __launch_bounds__(LK_THREADS) void k_lk_sort(
    const void* __restrict__ values, uint32_t n, const RowState* __restrict__ states,
    CallState* __restrict__ cs, const uint64_t* __restrict__ cbuf, uint64_t* __restrict__ aux,
    uint64_t* __restrict__ scratch, uint32_t cap, uint32_t k, uint32_t B, uint32_t bl,
    const uint32_t* __restrict__ lkc, void* __restrict__ out_values,
    int64_t* __restrict__ out_idx) {
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
  const uint32_t w0 = blockIdx.x * LK_WIN;
  if (w0 >= k) return;
  const uint32_t w1 = w0 + LK_WIN < k ? w0 + LK_WIN : k;
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
  uint64_t* A = aux + (size_t)row * cap;
  uint64_t* S = scratch + (size_t)row * cap;
  const LkDigit g = lk_digit_of(st, B, bl);

  // Bucket starts: start(r) = the sum over the row's chunks of their prefix
  // counts at rank r (start(LK_BINS) = R).  The window's buckets are the
  // ranks [rho(w0), rho(x1)), x1 = min(w1, R), with rho(x) = the least rank
  // whose bucket starts at or after x.  Two rounds of 64 probes find each
  // rho: every 64th rank (from the chunks' coarse copies), then the 64 ranks
  // of the step that holds it.  Lane i holds probe i and the waves share out
  // the chunks, so each load is 64 consecutive words of one chunk.
  // Invariant per bound x > 0: start(lo) < x <= start(hi).
  if (w0 >= R) return;   // (a row that keeps fewer than k: nothing starts here)
  const uint32_t nch = (R + LK_CHUNK - 1) / LK_CHUNK, maxch = lk_maxch(cap);
  const uint32_t* lkr = lkc + (size_t)row * maxch * LK_CSTRIDE;
  const uint32_t x1 = w1 < R ? w1 : R;
  constexpr uint32_t NW = LK_THREADS / 64;
  __shared__ uint32_t s_bnd[2][4];   // per bound: lo, hi, start(lo), start(hi)
  __shared__ uint32_t s_part[NW][64];
  __shared__ uint32_t s_pv[2][64];
  if (tid < 2) {
    s_bnd[tid][0] = 0u;
    s_bnd[tid][1] = LK_BINS;
    s_bnd[tid][2] = 0u;
    s_bnd[tid][3] = R;
  }
  auto clen = [&](uint32_t c) { return R - c * LK_CHUNK < LK_CHUNK ? R - c * LK_CHUNK : LK_CHUNK; };
  // for bound bd, by one wave: the first probe at or above it (probes at lo
  // + step (i + 1), their starts in s_pv[pv][i], non-decreasing in i, so the
  // probes below the bound are a prefix; the last probe is never below it)
  auto narrow = [&](uint32_t bd, uint32_t pv, uint32_t step) {
    const uint32_t x = bd == 0 ? w0 : x1;
    uint32_t i = (uint32_t)__builtin_popcountll(ballot(s_pv[pv][lane] < x));
    if (i > 63) i = 63;
    if (lane == 0) {
      const uint32_t lo = s_bnd[bd][0];
      if (i > 0) s_bnd[bd][2] = s_pv[pv][i - 1];
      s_bnd[bd][0] = lo + step * i;
      s_bnd[bd][1] = lo + step * (i + 1);
      s_bnd[bd][3] = s_pv[pv][i];
    }
  };
  // one lane's sum over the chunks c0, c0 + dc, ... of word `word` of each
  // chunk (LK_BINS + 1 meaning the chunk's length), eight loads in flight at
  // a time
  auto chunk_sum = [&](uint32_t c0, uint32_t dc, uint32_t word) {
    uint32_t part = 0;
    for (uint32_t cb = c0; cb < nch; cb += 8 * dc) {
      uint32_t v[8];
#pragma unroll
      for (uint32_t q = 0; q < 8; ++q) {
        const uint32_t c = cb + q * dc;
        v[q] = (c < nch && word <= LK_CSTRIDE - 1) ? lkr[(size_t)c * LK_CSTRIDE + word] : 0u;
      }
#pragma unroll
      for (uint32_t q = 0; q < 8; ++q) {
        const uint32_t c = cb + q * dc;
        if (c < nch) {
          const uint32_t len = clen(c);
          const uint32_t x = word <= LK_CSTRIDE - 1 ? v[q] : len;
          part += x < len ? x : len;
        }
      }
    }
    return part;
  };
  {   // round 1: ranks 64 (i + 1), the same probes for both bounds
    // (rank 64 m is word LK_BINS + m of a chunk; rank LK_BINS its length)
    const uint32_t part = chunk_sum(w, NW, lane < 63 ? LK_BINS + lane + 1 : LK_CSTRIDE);
    s_part[w][lane] = part;
    __syncthreads();
    if (w == 0) {
      uint32_t sm = 0;
      for (uint32_t q = 0; q < NW; ++q) sm += s_part[q][lane];
      s_pv[0][lane] = sm;
    }
    __syncthreads();
    if (w < 2) narrow(w, 0, 64);
    __syncthreads();
  }
  {   // round 2: the 64 ranks after each bound's lo; wave w: bound w & 1,
      // chunks w / 2, w / 2 + NW / 2, ...
    const uint32_t bd = w & 1u, r = s_bnd[bd][0] + 1 + lane;   // r <= LK_BINS
    const uint32_t part = chunk_sum(w >> 1, NW / 2, r < LK_BINS ? r : LK_CSTRIDE);
    s_part[w][lane] = part;
    __syncthreads();
    if (w < 2) {
      uint32_t sm = 0;
      for (uint32_t q = w; q < NW; q += 2) sm += s_part[q][lane];
      s_pv[w][lane] = sm;
    }
    __syncthreads();
    if (w < 2) narrow(w, w, 1);
    __syncthreads();
  }
  // rho(0) = 0 (the first window's lower bound; the search assumes x > 0)
  const uint32_t r_lo = w0 == 0 ? 0u : s_bnd[0][1];
  const uint32_t a0s = w0 == 0 ? 0u : s_bnd[0][3];
  const uint32_t r_end = s_bnd[1][1], e0s = s_bnd[1][3], lasts = s_bnd[1][2];
  if (r_lo >= r_end) return;   // no bucket starts in this window
  const uint32_t r_last = r_end - 1;
  // the window's candidates fit one LDS sort (the common case): gathered
  // straight into LDS; otherwise into aux, for the split
  const bool in_lds = e0s - a0s <= LK_LCAP;
  __syncthreads();   // every thread has read the bounds

  // Gather: chunk c holds ranks [r_lo, r_last) as one run and rank r_last
  // right after it; the runs of the chunks in chunk order go to A[a0, last)
  // and A[last, e0) as v values (one thread per chunk finds its runs, a
  // prefix over the chunks places them, then every thread copies).
  {
    __shared__ uint32_t s_hp[LK_MAXCH + 1], s_tp[LK_MAXCH + 1], s_lo[LK_MAXCH], s_mid[LK_MAXCH];
    __shared__ uint32_t s_ws[2 * (LK_THREADS / 64)];
    static_assert(LK_MAXCH <= LK_THREADS, "one thread per chunk");
    uint32_t hd = 0, tl = 0, lo = 0, mid = 0;
    if (tid < nch) {
      const uint32_t* pc = lkc + ((size_t)row * maxch + tid) * LK_CSTRIDE;
      const uint32_t len = R - tid * LK_CHUNK < LK_CHUNK ? R - tid * LK_CHUNK : LK_CHUNK;
      lo = pc[r_lo];
      mid = pc[r_last];
      uint32_t hi = r_end < LK_BINS ? pc[r_end] : len;
      // (prefix counts never exceed the chunk; clamped all the same)
      hi = hi < len ? hi : len;
      mid = mid < hi ? mid : hi;
      lo = lo < mid ? lo : mid;
      hd = mid - lo;
      tl = hi - mid;
    }
    const uint32_t ih = wave_incl_sum(hd), it = wave_incl_sum(tl);
    if (lane == 63) {
      s_ws[w] = ih;
      s_ws[LK_THREADS / 64 + w] = it;
    }
    __syncthreads();
    uint32_t ph = ih - hd, pt = it - tl;
    for (uint32_t i = 0; i < nt / 64; ++i) {
      ph += i < w ? s_ws[i] : 0u;
      pt += i < w ? s_ws[LK_THREADS / 64 + i] : 0u;
    }
    if (tid < nch) {
      s_hp[tid] = ph;
      s_tp[tid] = pt;
      s_lo[tid] = tid * LK_CHUNK + lo;
      s_mid[tid] = tid * LK_CHUNK + mid;
    }
    if (tid == nch - 1) {
      s_hp[nch] = ph + hd;
      s_tp[nch] = pt + tl;
    }
    __syncthreads();
    const uint32_t a0 = a0s, last = lasts;
    const uint64_t* cb = cbuf + (size_t)row * cap;
    // the chunk holding gathered element i: the last c with s_p[c] <= i
    auto chunk_of = [&](const uint32_t* s_p, uint32_t i) {
      uint32_t lo_c = 0, hi_c = nch;   // s_p[lo_c] <= i < s_p[hi_c]
      while (hi_c - lo_c > 1) {
        const uint32_t m = (lo_c + hi_c) >> 1;
        if (s_p[m] <= i) lo_c = m;
        else hi_c = m;
      }
      return lo_c;
    };
    // (equal to last - a0 and e0 - last when the chunks and the histogram
    // agree, as they always do; bounded by them all the same)
    const uint32_t e0c = e0s < cap ? e0s : cap;
    const uint32_t H = s_hp[nch] < last - a0 ? s_hp[nch] : last - a0;
    const uint32_t T = last < e0c ? (s_tp[nch] < e0c - last ? s_tp[nch] : e0c - last) : 0u;
    for (uint32_t i = tid; i < H; i += nt) {
      const uint32_t c = chunk_of(s_hp, i);
      const uint64_t v = g.compact(cb[s_lo[c] + (i - s_hp[c])]);
      if (in_lds) s_a[i] = v;
      else A[a0 + i] = v;
    }
    for (uint32_t i = tid; i < T; i += nt) {
      const uint32_t c = chunk_of(s_tp, i);
      const uint64_t v = g.compact(cb[s_mid[c] + (i - s_tp[c])]);
      if (in_lds) s_a[(last - a0) + i] = v;
      else A[last + i] = v;
    }
    __syncthreads();   // the gathered values are visible to the workgroup
  }

  // sort [lo, lo + len) of src (compacted values, unique, len <= LK_LCAP; src
  // null: they are in s_a already) in LDS and write the output positions
  // below k.  nb > 0: the range is the
  // buckets of ranks r_last - nb + 1 .. r_last, and the sort's bins are the
  // bucket and the bits just below the bucket digit; nb = 0: bins from the
  // range's extremes.
  auto sort_out = [&](const uint64_t* src, uint32_t lo, uint32_t len, uint32_t nb,
                      uint32_t r_last) {
    if (src) {   // (null: the range is in s_a already)
      for (uint32_t i = tid; i < len; i += nt) s_a[i] = src[lo + i];
      __syncthreads();
    }
    bool ok;
    if (nb > 0 && nb <= 2048) {
      uint32_t sb = 31u - (uint32_t)__builtin_clz(2048u / nb);   // nb << sb <= 2048
      if (sb > g.shift) sb = g.shift;
      const uint32_t dsh = g.shift - sb;
      const uint64_t dbase = (uint64_t)(LK_BINS - 1 - r_last) << sb;
      ok = block_sort_binned_desc(s_a, len, s_b, s_hist, s_sm, reinterpret_cast<uint32_t*>(s_red),
                                  [&](uint64_t v) { return (uint32_t)((v >> dsh) - dbase); }, 64u);
    } else if (nb > 2048) {
      // more buckets than bins (the first windows, where the largest keys are
      // sparse): 2^sm neighbouring buckets per bin
      uint32_t sm = 1;
      while (((nb - 1) >> sm) >= 2048u) ++sm;
      const uint64_t dbase = (uint64_t)(LK_BINS - 1 - r_last);
      ok = block_sort_binned_desc(s_a, len, s_b, s_hist, s_sm, reinterpret_cast<uint32_t*>(s_red),
                                  [&](uint64_t v) { return (uint32_t)(((v >> g.shift) - dbase) >> sm); },
                                  64u);
      if (!ok) ok = block_sort_unique_desc(s_a, len, s_b, s_hist, s_sm, s_red, 64u);
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

  const uint32_t a0 = a0s, e0 = e0s, last = lasts;
  if (in_lds) {
    sort_out(nullptr, a0, e0 - a0, r_end - r_lo, r_end - 1);
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
