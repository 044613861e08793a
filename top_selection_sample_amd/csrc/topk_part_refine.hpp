// Refinement: ranking and output writers, refine_row, refine_sampled, the one-workgroup route (k_exact_small).
// A part of topk_kernels.hip, included there in order inside namespace tk;
// it relies on the definitions of the parts before it and is not a
// stand-alone header.
#pragma once

// ======================================================================
// Refinement (Prof-K section 3, stage 4): exact top-k of the candidate
// buffer, one workgroup per row: radix select of the k-th composite, gather
// of the k winners, bitonic sort into rank order, and the output write
// (values are re-read from the input so they keep their own bits).
// ======================================================================
struct CompSrc {
  const uint64_t* p;
  __device__ uint64_t operator()(uint32_t i) const { return p[i]; }
};

template <int DT>
struct RowSrc {
  const char* rowp;
  uint32_t B;
  uint64_t maskB;
  __device__ uint64_t operator()(uint32_t i) const {
    return ((uint64_t)Dt<DT>::key(load_raw<DT>(rowp, i)) << B) | (maskB - i);
  }
};

// The output value of a winner: the input element's own bits.  They follow
// from the key except for +-0 and NaN, which are read from the input.
template <int DT>
__device__ __forceinline__ uint32_t winner_bits(uint64_t c, uint32_t B, const char* rowp,
                                                uint32_t n, uint32_t* idx_out) {
  const uint64_t maskB = (1ull << B) - 1ull;
  uint32_t idx = (uint32_t)(maskB - (c & maskB));
  if (idx >= n) idx = n - 1;   // only a padding entry could decode out of range
  *idx_out = idx;
  uint32_t bits;
  if (Dt<DT>::unkey((uint32_t)(c >> B), &bits)) return bits;
  return load_raw<DT>(rowp, idx);
}

template <int DT>
__device__ __forceinline__ void store_winner(void* out_values, int64_t* out_idx, size_t o,
                                             uint32_t bits, uint32_t idx) {
  if constexpr (DT == DT_BF16) static_cast<uint16_t*>(out_values)[o] = (uint16_t)bits;
  else static_cast<uint32_t*>(out_values)[o] = bits;
  out_idx[o] = idx;
}

// Output slot of s[i] = #{j : s[j] > s[i]}; slots >= k are dropped, and a
// row's slots start at row * ks.  Four neighbouring lanes share an element,
// each counting a quarter of the list; their counts are summed with two quad
// moves.  Needs cnt <= blockDim.x / 4 and every thread of the workgroup.
template <int DT>
__device__ void rank_and_write(const uint64_t* s, uint32_t cnt, uint32_t k, uint32_t ks,
                               uint32_t B, const char* rowp, uint32_t n, void* out_values,
                               int64_t* out_idx, uint32_t row) {
  const uint32_t i = threadIdx.x >> 2, q = threadIdx.x & 3u;
  if (((threadIdx.x & ~63u) >> 2) >= cnt) return;   // a wave with no element (uniform)
  const uint64_t c = i < cnt ? s[i] : ~0ull;
  uint32_t r0 = 0, r1 = 0;
  uint32_t j = q;
  for (; j + 4 < cnt; j += 8) {   // two independent LDS reads per step
    r0 += (s[j] > c) ? 1u : 0u;
    r1 += (s[j + 4] > c) ? 1u : 0u;
  }
  if (j < cnt) r0 += (s[j] > c) ? 1u : 0u;
  uint32_t r = r0 + r1;
  r += dpp_take<0xB1, 0xf>(r);   // lanes 1,0,3,2 of each quad
  r += dpp_take<0x4E, 0xf>(r);   // lanes 2,3,0,1
  if (q == 0 && i < cnt && r < k) {
    uint32_t idx;
    const uint32_t bits = winner_bits<DT>(c, B, rowp, n, &idx);
    store_winner<DT>(out_values, out_idx, (size_t)row * ks + r, bits, idx);
  }
}

// The first k of the sorted list s_w to the row's slots (which start at
// row * ks).
template <int DT>
__device__ void write_winners(const uint64_t* s_w, uint32_t k, uint32_t ks, uint32_t B,
                              const char* rowp, uint32_t n, void* out_values, int64_t* out_idx,
                              uint32_t row) {
  for (uint32_t i = threadIdx.x; i < k; i += blockDim.x) {
    uint32_t idx;
    const uint32_t bits = winner_bits<DT>(s_w[i], B, rowp, n, &idx);
    store_winner<DT>(out_values, out_idx, (size_t)row * ks + i, bits, idx);
  }
}

// An output slot no winner fills (a row that keeps fewer than k): index -1
// and the dtype's lowest value (-inf for the floats, INT32_MIN for int32).
template <int DT>
__device__ __forceinline__ void store_pad(void* out_values, int64_t* out_idx, size_t o) {
  if constexpr (DT == DT_BF16) static_cast<uint16_t*>(out_values)[o] = 0xFF80u;
  else static_cast<uint32_t*>(out_values)[o] = DT == DT_I32 ? 0x80000000u : 0xFF800000u;
  out_idx[o] = -1;
}

// Slots [from, ks) of the row, padded.
template <int DT>
__device__ void pad_slots(uint32_t from, uint32_t ks, void* out_values, int64_t* out_idx,
                          uint32_t row) {
  for (uint32_t i = from + threadIdx.x; i < ks; i += blockDim.x)
    store_pad<DT>(out_values, out_idx, (size_t)row * ks + i);
}

// s_tmp: 16 words (at most 1024 threads).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* s_tmp) {
  v = wave_max_u32(v);
  if ((threadIdx.x & 63u) == 0) s_tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t nw = blockDim.x >> 6;
  uint32_t m = 0;
#pragma unroll
  for (uint32_t j = 0; j < 16; ++j) {   // independent reads
    const uint32_t x = j < nw ? s_tmp[j] : 0u;
    m = x > m ? x : m;
  }
  __syncthreads();
  return m;
}

constexpr uint32_t RF_BITS = 11;
constexpr uint32_t RF_BINS = 1u << RF_BITS;
constexpr uint32_t RF_SORT_CAP = 4096;
constexpr uint32_t RF_KCAP = 24576;     // candidate keys cached in LDS (96 KB)
constexpr uint32_t RF_RANK_MAX = 256;   // up to this many: rank counting, else bitonic

// Sort s[0..cnt) descending in LDS (cnt <= CAND_CAP), zero-padded to a power
// of two; composites are never zero, so padding sorts last.
__device__ __forceinline__ void lds_sort_desc(uint64_t* s, uint32_t cnt) {
  const uint32_t P = next_pow2(cnt);
  for (uint32_t i = cnt + threadIdx.x; i < P; i += blockDim.x) s[i] = 0ull;
  __syncthreads();
  block_bitonic_desc(s, P);
}

// The k largest of the `got` unique composites in s_cand (got >= k) to the
// output, in rank order; the row's slots start at row * ks (ks >= k).  tmp: LDS scratch of 2 * RF_SORT_CAP + 64 words.
// digit: a bin of 11 key bits that never decreases as the composite grows,
// or null to take one from the list's own range.
template <int DT, class Digit>
__device__ void emit_winners(const void* __restrict__ values, uint32_t n, uint32_t k, uint32_t ks,
                             uint32_t B, void* __restrict__ out_values, int64_t* __restrict__ out_idx,
                             uint32_t row, uint64_t* s_cand, uint32_t got, uint32_t* s_hist,
                             uint32_t* s_misc, uint64_t* tmp, const Digit* digit) {
  const uint32_t tid = threadIdx.x;
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
  if (got <= RF_RANK_MAX) {
    // few elements: each one's output slot is the number of larger
    // composites (the rank of GPU.js Learn "Rank by Counting"; composites are
    // unique, so the slots are a permutation)
    rank_and_write<DT>(s_cand, got, k, ks, B, rowp, n, out_values, out_idx, row);
  } else {
    uint32_t* wsum = reinterpret_cast<uint32_t*>(tmp + RF_SORT_CAP);
    bool sorted = digit && block_sort_binned_desc(s_cand, got, tmp, s_hist, s_misc, wsum, *digit, 64u);
    if (!sorted) sorted = block_sort_unique_desc(s_cand, got, tmp, s_hist, s_misc, tmp + RF_SORT_CAP, 64u);
    if (!sorted) {
      uint64_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t i = 4 * tid + (uint32_t)j;
        v[j] = i < got ? s_cand[i] : 0ull;
      }
      block_bitonic4096_desc(v, tmp);
#pragma unroll
      for (int j = 0; j < 4; ++j) s_cand[4 * tid + j] = v[j];
      __syncthreads();
    }
    write_winners<DT>(s_cand, k, ks, B, rowp, n, out_values, out_idx, row);
  }
}

struct NoDigit {
  __device__ uint32_t operator()(uint64_t) const { return 0u; }
};

// One row, one workgroup (1024 threads): the exact route's candidates
// (want = ST_EXACT_READY; the sampled route's rows use refine_sampled).
// A key pass fills an LDS key cache and finds the largest key, the
// histogram and the boundary bin come from the cache, and the candidates
// from the boundary bin up are gathered from the buffer.
template <int DT>
__device__ void refine_row(const void* __restrict__ values, uint32_t n, RowState* __restrict__ states,
                           CallState* cs, uint32_t* flagged, const uint64_t* __restrict__ cbuf,
                           uint32_t cap, uint32_t k, uint32_t B, uint32_t W, uint32_t want,
                           void* __restrict__ out_values, int64_t* __restrict__ out_idx,
                           uint32_t row, uint32_t* s_hist, uint32_t* s_misc, uint32_t* s_tmp,
                           uint64_t* s_cand, uint32_t* s_keys, uint32_t* s_idx) {
  // LDS: s_hist[RF_BINS], s_misc[8], s_tmp[16], s_cand[RF_SORT_CAP],
  //      s_keys[RF_KCAP], s_idx[RF_SORT_CAP]
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  RowState* st = states + row;
  if (st->status != want) return;
  uint32_t R = st->count;   // in [k, cap]: the row passed its check
  if (R > cap) R = cap;
  const uint32_t KB = W - B;
  const uint32_t lo_key = (want == ST_FILTER) ? st->tau_key : st->thr_key;
  CompSrc src{cbuf + (size_t)row * cap};

  // Pass 0 reads every candidate once: its key goes to the LDS key cache
  // (the first RF_KCAP), and the largest key is kept.
  const uint32_t Rc = R < RF_KCAP ? R : RF_KCAP;
  uint32_t mx = 0;
  for_batched_i<LOADS_IN_FLIGHT, uint64_t>(
      R, [&](uint32_t i) { return src.p[i]; },
      [&](uint64_t c, bool ok, uint32_t i) {
        const uint32_t key = ok ? (uint32_t)(c >> B) : 0u;
        if (ok && i < Rc) s_keys[i] = key;
        mx = key > mx ? key : mx;
      });
  const uint32_t kmax = block_max_u32(mx, s_tmp);   // (has the barrier the cache needs)
  // every candidate key lies in [lo_key, kmax]: histogram the 11 key bits
  // just below their common prefix
  const uint32_t diff = (lo_key ^ kmax) & (KB == 32 ? 0xFFFFFFFFu : 0xFFFFu);
  const uint32_t top = diff ? 31u - (uint32_t)__builtin_clz(diff) : 0u;
  const uint32_t kshift = top >= RF_BITS - 1 ? top - (RF_BITS - 1) : 0u;
  auto digit = [&](uint32_t key) { return (key >> kshift) & (RF_BINS - 1); };
  for (uint32_t i = tid; i < RF_BINS; i += nt) s_hist[i] = 0;
  __syncthreads();
  {
    uint32_t i = tid;
    for (; i + 3 * nt < Rc; i += 4 * nt) {   // four independent LDS reads per step
      const uint32_t k0 = s_keys[i], k1 = s_keys[i + nt], k2 = s_keys[i + 2 * nt],
                     k3 = s_keys[i + 3 * nt];
      atomicAdd(&s_hist[digit(k0)], 1u);
      atomicAdd(&s_hist[digit(k1)], 1u);
      atomicAdd(&s_hist[digit(k2)], 1u);
      atomicAdd(&s_hist[digit(k3)], 1u);
    }
    for (; i < Rc; i += nt) atomicAdd(&s_hist[digit(s_keys[i])], 1u);
  }
  if (R > Rc)
    for_batched<LOADS_IN_FLIGHT, uint64_t>(
        R - Rc, [&](uint32_t i) { return src.p[Rc + i]; },
        [&](uint64_t c, bool ok) { hist_add(s_hist, digit((uint32_t)(c >> B)), ok); });
  __syncthreads();
  block_find_bucket(s_hist, RF_BINS, k, s_misc, s_tmp);
  const uint32_t b = s_misc[0], acc = s_misc[1], hb = s_misc[2];
  __syncthreads();
  uint32_t got;
  if (acc + hb <= RF_SORT_CAP) {
    // pass 2: list the indices at or above the boundary bucket, then gather
    // those composites and sort them in LDS
    if (tid == 0) s_misc[4] = 0;
    __syncthreads();
    for (uint32_t i0 = 0; i0 < Rc; i0 += nt) {
      const uint32_t i = i0 + tid;
      const bool keep = i < Rc && digit(s_keys[i]) >= b;
      lds_append_u32(s_idx, &s_misc[4], RF_SORT_CAP, i, keep);
    }
    if (R > Rc)
      for_batched_i<LOADS_IN_FLIGHT, uint64_t>(
          R - Rc, [&](uint32_t i) { return src.p[Rc + i]; },
          [&](uint64_t c, bool ok, uint32_t i) {
            lds_append_u32(s_idx, &s_misc[4], RF_SORT_CAP, Rc + i,
                           ok && digit((uint32_t)(c >> B)) >= b);
          });
    __syncthreads();
    got = s_misc[4] < RF_SORT_CAP ? s_misc[4] : RF_SORT_CAP;
    for_batched_i<4, uint64_t>(
        got, [&](uint32_t j) { return src.p[s_idx[j]]; },
        [&](uint64_t c, bool ok, uint32_t j) {
          if (ok) s_cand[j] = c;
        });
    __syncthreads();
  } else {
    // heavy ties or a wide boundary bucket: radix select on the composite
    SelectOut sel = block_select(src, R, W, k, k, s_hist, s_misc, s_cand, RF_SORT_CAP);
    got = block_collect(src, R, sel.thr, s_cand, RF_SORT_CAP, &s_misc[4]);
  }
  emit_winners<DT, NoDigit>(values, n, k, k, B, out_values, out_idx, row, s_cand, got, s_hist, s_misc,
                            reinterpret_cast<uint64_t*>(s_keys), nullptr);
  __syncthreads();
  if (tid == 0) st->status = ST_DONE;
  __syncthreads();
}

// The sampled route's refine (Prof-K section 3, stage 4: the exact top-k of
// the candidates), one row per workgroup of RS_THREADS.  The candidates are
// read from global memory once and stay in registers (RS_VEC pairs per
// thread; a longer buffer streams its remainder).  Their keys lie in
// [tau, kmax], kmax being the largest key the filter stored, so the 11 key
// bits just below the common prefix of tau and kmax order them: one LDS
// histogram finds the bin holding rank k, and the candidates from that bin
// up go straight from registers to LDS for the final rank or sort.  The k
// winners fill the row's first k slots of ks; a row that keeps fewer than ks
// (k = R) gets the rest padded.
constexpr uint32_t RS_VEC = 11;
constexpr uint32_t RS_THREADS = 1024;
template <int DT>
__device__ void refine_sampled(const void* __restrict__ values, uint32_t n, RowState* st,
                               const uint64_t* __restrict__ cb, uint32_t R, uint32_t lo,
                               uint32_t kmax, uint32_t k, uint32_t ks, uint32_t B, uint32_t W,
                               void* __restrict__ out_values, int64_t* __restrict__ out_idx,
                               uint32_t row, uint32_t* s_hist, uint32_t* s_misc, uint32_t* s_tmp,
                               uint64_t* s_cand, uint64_t* s_scratch) {
  const uint32_t tid = threadIdx.x, nt = RS_THREADS;
  const uint32_t KB = W - B;
  const uint32_t hi = kmax > lo ? kmax : lo;
  const uint32_t diff = (lo ^ hi) & (KB == 32 ? 0xFFFFFFFFu : 0xFFFFu);
  const uint32_t top = diff ? 31u - (uint32_t)__builtin_clz(diff) : 0u;
  const uint32_t kshift = top >= RF_BITS - 1 ? top - (RF_BITS - 1) : 0u;
  auto digit = [&](uint64_t c) { return ((uint32_t)(c >> B) >> kshift) & (RF_BINS - 1); };

  // Issue every load first.  The row's buffer starts 8-byte aligned: an odd
  // start leaves one leading composite to thread 0, then come 16-byte pairs,
  // and an odd last one goes to thread 1.  Candidates beyond the registers
  // are streamed.
  const uint32_t nh = (R && ((reinterpret_cast<uintptr_t>(cb) >> 3) & 1u)) ? 1u : 0u;
  const uint32_t pairs = (R - nh) / 2;
  const uint32_t nvr = pairs < RS_VEC * nt ? pairs : RS_VEC * nt;
  const uint32_t tl = (nvr == pairs && ((R - nh) & 1u)) ? 1u : 0u;
  const uint32_t r0 = nh + 2 * nvr, re = R - tl;   // the streamed range [r0, re)
  const u64x2* vp = reinterpret_cast<const u64x2*>(cb + nh);
  u64x2 x[RS_VEC];
#pragma unroll
  for (uint32_t j = 0; j < RS_VEC; ++j) {
    const uint32_t v = j * nt + tid;
    x[j] = v < nvr ? __builtin_nontemporal_load(vp + v) : u64x2{0ull, 0ull};
  }
  const bool has1 = (tid == 0 && nh) || (tid == 1 && tl);
  const uint64_t x1 = has1 ? cb[tid == 0 ? 0u : R - 1] : 0ull;
  for (uint32_t i = tid; i < RF_BINS; i += nt) s_hist[i] = 0;
  if (tid == 0) s_misc[4] = 0;
  __syncthreads();
  hist_add(s_hist, digit(x1), has1);
#pragma unroll
  for (uint32_t j = 0; j < RS_VEC; ++j) {
    const bool ok = j * nt + tid < nvr;
    hist_add(s_hist, digit(x[j].x), ok);
    hist_add(s_hist, digit(x[j].y), ok);
  }
  if (r0 < re)
    for_batched<LOADS_IN_FLIGHT, uint64_t>(
        re - r0, [&](uint32_t i) { return cb[r0 + i]; },
        [&](uint64_t c, bool ok) { hist_add(s_hist, digit(c), ok); });
  __syncthreads();
  block_find_bucket_2048<RS_THREADS>(s_hist, k, s_misc, s_tmp);
  __syncthreads();
  const uint32_t b = s_misc[0], acc = s_misc[1], hb = s_misc[2];
  uint32_t got;
  if (acc + hb <= RF_SORT_CAP) {
    // the register-held ones: one slot reservation per wave
    auto keep = [&](uint64_t c, bool ok) { return ok && digit(c) >= b; };
    uint32_t mine = keep(x1, has1) ? 1u : 0u;
#pragma unroll
    for (uint32_t j = 0; j < RS_VEC; ++j) {
      const bool ok = j * nt + tid < nvr;
      mine += (keep(x[j].x, ok) ? 1u : 0u) + (keep(x[j].y, ok) ? 1u : 0u);
    }
    const uint32_t incl = wave_incl_sum(mine);
    const uint32_t wtot = wave_bcast(incl, 63u);
    uint32_t wbase = 0;
    if ((tid & 63u) == 0 && wtot) wbase = atomicAdd(&s_misc[4], wtot);
    uint32_t pos = wave_bcast(wbase, 0u) + incl - mine;
    auto put = [&](uint64_t c, bool k) {
      if (k) {
        if (pos < RF_SORT_CAP) s_cand[pos] = c;
        ++pos;
      }
    };
    put(x1, keep(x1, has1));
#pragma unroll
    for (uint32_t j = 0; j < RS_VEC; ++j) {
      const bool ok = j * nt + tid < nvr;
      put(x[j].x, keep(x[j].x, ok));
      put(x[j].y, keep(x[j].y, ok));
    }
    if (r0 < re)
      for_batched<LOADS_IN_FLIGHT, uint64_t>(
          re - r0, [&](uint32_t i) { return cb[r0 + i]; },
          [&](uint64_t c, bool ok) {
            lds_append(s_cand, &s_misc[4], RF_SORT_CAP, c, ok && digit(c) >= b);
          });
    __syncthreads();
    got = s_misc[4] < RF_SORT_CAP ? s_misc[4] : RF_SORT_CAP;
  } else {
    // heavy ties or a wide boundary bin: radix select on the composite
    __syncthreads();   // every thread has read the bin
    CompSrc src{cb};
    SelectOut sel = block_select(src, R, W, k, k, s_hist, s_misc, s_cand, RF_SORT_CAP);
    got = block_collect(src, R, sel.thr, s_cand, RF_SORT_CAP, &s_misc[4]);
  }
  // the collected candidates keep the histogram's bins: sort on them
  struct BinOf {
    uint32_t B, kshift;
    __device__ uint32_t operator()(uint64_t c) const {
      return ((uint32_t)(c >> B) >> kshift) & (RF_BINS - 1);
    }
  } bin_of{B, kshift};
  emit_winners<DT, BinOf>(values, n, k, ks, B, out_values, out_idx, row, s_cand, got, s_hist,
                          s_misc, s_scratch, &bin_of);
  if (k < ks) pad_slots<DT>(k, ks, out_values, out_idx, row);
  __syncthreads();
  if (tid == 0) st->status = ST_DONE;
  __syncthreads();
}

// A short row (n <= NV * blockDim.x) and k <= RF_RANK_MAX: the row is
// read once into registers; a block min and max of its keys give the 11 key
// bits just below their common prefix, whose LDS histogram finds the bin
// holding rank k; the elements from that bin up go to LDS and, when there
// are at most RF_RANK_MAX of them, are ranked by counting and written.
// Returns false, having written nothing, when more elements reach that bin
// (heavy ties); the caller then runs the radix select.  s_tmp: 32 words;
// s_hist2048: RF_BINS words, 16-byte aligned, apart from s_cand[0 ..
// RF_RANK_MAX).  Every thread of the workgroup calls it.
template <int DT, uint32_t NV>
__device__ bool exact_row_in_registers(const char* rowp, uint32_t n, uint32_t k, uint32_t B,
                                       void* out_values, int64_t* out_idx, uint32_t row,
                                       uint32_t* s_tmp, uint32_t* s_misc, uint32_t* s_hist2048,
                                       uint64_t* s_cand) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x, lane = tid & 63u, w = tid >> 6;
  uint32_t key[NV];
  uint32_t mx = 0, mn = 0xFFFFFFFFu;
#pragma unroll
  for (uint32_t j = 0; j < NV; ++j) {
    const uint32_t i = j * nt + tid;
    key[j] = i < n ? Dt<DT>::key(load_raw<DT>(rowp, i)) : 0u;
    if (i < n) {
      mx = key[j] > mx ? key[j] : mx;
      mn = key[j] < mn ? key[j] : mn;
    }
  }
  for (uint32_t i = tid; i < RF_BINS; i += nt) s_hist2048[i] = 0;
  if (tid == 0) s_misc[4] = 0;
  mx = wave_max_u32(mx);
  mn = ~wave_max_u32(~mn);
  if (lane == 0) {
    s_tmp[w] = mx;
    s_tmp[16 + w] = mn;
  }
  __syncthreads();
  const uint32_t nw = nt >> 6;
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (uint32_t j = 0; j < 16; ++j) {   // independent reads
    const uint32_t a = j < nw ? s_tmp[j] : 0u, c = j < nw ? s_tmp[16 + j] : 0xFFFFFFFFu;
    kmax = a > kmax ? a : kmax;
    kmin = c < kmin ? c : kmin;
  }
  const uint32_t diff = kmin ^ kmax;
  const uint32_t top = diff ? 31u - (uint32_t)__builtin_clz(diff) : 0u;
  const uint32_t kshift = top >= RF_BITS - 1 ? top - (RF_BITS - 1) : 0u;
  auto digit = [&](uint32_t x) { return (x >> kshift) & (RF_BINS - 1); };
#pragma unroll
  for (uint32_t j = 0; j < NV; ++j) hist_add(s_hist2048, digit(key[j]), j * nt + tid < n);
  __syncthreads();
  if (tid < 64) wave_find_bucket_2048(s_hist2048, k, s_misc);
  __syncthreads();
  const uint32_t b = s_misc[0], got = s_misc[1] + s_misc[2];
  if (got > RF_RANK_MAX) return false;   // (uniform)
  // the elements from the bin up, one slot reservation per wave
  const uint64_t maskB = (1ull << B) - 1ull;
  uint32_t mine = 0;
#pragma unroll
  for (uint32_t j = 0; j < NV; ++j) mine += (j * nt + tid < n && digit(key[j]) >= b) ? 1u : 0u;
  const uint32_t incl = wave_incl_sum(mine);
  const uint32_t wtot = wave_bcast(incl, 63u);
  uint32_t wbase = 0;
  if (lane == 0 && wtot) wbase = atomicAdd(&s_misc[4], wtot);
  uint32_t pos = wave_bcast(wbase, 0u) + incl - mine;
#pragma unroll
  for (uint32_t j = 0; j < NV; ++j) {
    const uint32_t i = j * nt + tid;
    if (i < n && digit(key[j]) >= b) s_cand[pos++] = ((uint64_t)key[j] << B) | (maskB - i);
  }
  __syncthreads();
  rank_and_write<DT>(s_cand, got, k, k, B, rowp, n, out_values, out_idx, row);
  return true;
}

// The same for rows too long for the registers (n <= ER_STREAM_MAX): three
// reads of the row in 16-byte vectors (its key range, the histogram, the
// collection), the last two from L2.  values: the whole input (the row's
// unaligned head and tail elements are visited by the first wave).
constexpr uint32_t ER_STREAM_MAX = 1u << 16;
template <int DT>
__device__ bool exact_row_streamed(const void* values, uint32_t n, uint32_t k, uint32_t B,
                                   void* out_values, int64_t* out_idx, uint32_t row,
                                   uint32_t* s_tmp, uint32_t* s_misc, uint32_t* s_hist2048,
                                   uint64_t* s_cand) {
  using D = Dt<DT>;
  constexpr uint32_t U = 4;               // 16-byte loads in flight per thread
  constexpr uint32_t E = U * D::VEC;      // elements per thread per step
  const uint32_t tid = threadIdx.x, nt = blockDim.x, lane = tid & 63u, w = tid >> 6;
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * D::ES;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(rowp);
  uint32_t head = (uint32_t)(((16u - (addr & 15u)) & 15u) / D::ES);
  if (head > n) head = n;
  const uint32_t nvec = (n - head) / D::VEC;
  const uint32_t tail0 = head + nvec * D::VEC;
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + (size_t)head * D::ES);
  // f(key, index, valid) for every element; every thread calls it the same
  // number of times within a wave, so f may use wave operations
  auto visit = [&](auto&& f) {
    for (uint32_t v0 = 0; v0 < nvec; v0 += U * nt) {
      u32x4 x[U];
#pragma unroll
      for (uint32_t j = 0; j < U; ++j) {
        const uint32_t v = v0 + j * nt + tid;
        x[j] = v < nvec ? vp[v] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (uint32_t b = 0; b < E; ++b) {
        const uint32_t v = v0 + (b / D::VEC) * nt + tid;
        f(D::key(elemvc<DT, U>(x, b)), head + v * D::VEC + b % D::VEC, v < nvec);
      }
    }
    if (tid < 64) {   // fewer than 2 * VEC elements outside the vectors
      const bool ok = tid < head + (n - tail0);
      uint32_t idx = 0, key = 0;
      if (ok) {
        idx = tid < head ? tid : tail0 + (tid - head);
        key = D::key(load_raw<DT>(rowp, idx));
      }
      f(key, idx, ok);
    }
  };
  uint32_t mx = 0, mn = 0xFFFFFFFFu;
  visit([&](uint32_t key, uint32_t, bool ok) {
    if (ok) {
      mx = key > mx ? key : mx;
      mn = key < mn ? key : mn;
    }
  });
  for (uint32_t i = tid; i < RF_BINS; i += nt) s_hist2048[i] = 0;
  if (tid == 0) s_misc[4] = 0;
  mx = wave_max_u32(mx);
  mn = ~wave_max_u32(~mn);
  if (lane == 0) {
    s_tmp[w] = mx;
    s_tmp[16 + w] = mn;
  }
  __syncthreads();
  const uint32_t nw = nt >> 6;
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (uint32_t j = 0; j < 16; ++j) {   // independent reads
    const uint32_t a = j < nw ? s_tmp[j] : 0u, c = j < nw ? s_tmp[16 + j] : 0xFFFFFFFFu;
    kmax = a > kmax ? a : kmax;
    kmin = c < kmin ? c : kmin;
  }
  const uint32_t diff = kmin ^ kmax;
  const uint32_t top = diff ? 31u - (uint32_t)__builtin_clz(diff) : 0u;
  const uint32_t kshift = top >= RF_BITS - 1 ? top - (RF_BITS - 1) : 0u;
  auto digit = [&](uint32_t x) { return (x >> kshift) & (RF_BINS - 1); };
  visit([&](uint32_t key, uint32_t, bool ok) { hist_add(s_hist2048, digit(key), ok); });
  __syncthreads();
  if (tid < 64) wave_find_bucket_2048(s_hist2048, k, s_misc);
  __syncthreads();
  const uint32_t b = s_misc[0], got = s_misc[1] + s_misc[2];
  if (got > RF_RANK_MAX) return false;   // (uniform)
  const uint64_t maskB = (1ull << B) - 1ull;
  visit([&](uint32_t key, uint32_t idx, bool ok) {
    lds_append(s_cand, &s_misc[4], RF_RANK_MAX, ((uint64_t)key << B) | (maskB - idx),
               ok && digit(key) >= b);
  });
  __syncthreads();
  rank_and_write<DT>(s_cand, got, k, k, B, rowp, n, out_values, out_idx, row);
  return true;
}

// Whole exact selection of a small row in one workgroup.  Small k: writes the
// answer.  Large k: leaves exactly k winners in the candidate buffer for the
// multi-workgroup sort.
template <int DT>
__global__ __launch_bounds__(SEL_THREADS) void k_exact_small(
    const void* __restrict__ values, uint32_t n, RowState* __restrict__ states,
    uint64_t* __restrict__ cbuf, uint32_t cap, uint32_t k, uint32_t B, uint32_t W,
    uint32_t small_k, void* __restrict__ out_values, int64_t* __restrict__ out_idx,
    CallState* cs, WsHeader* hdr, uint64_t sig) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_misc[8];
  __shared__ __align__(16) uint64_t s_cand[CAND_CAP];
  static_assert(CAND_CAP * 2 >= RF_RANK_MAX * 2 + RF_BINS, "bins beside the ranked candidates");
  const uint32_t row = blockIdx.x;
  RowState* st = states + row;
  // the call's set-up (this route's only kernel before the large-k sort):
  // the call record and the stamp
  if (row == 0 && threadIdx.x == 0) {
    reset_call(cs);
    stamp_invalidate(hdr, sig);
  }
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
  auto finish_row = [&]() {
    __syncthreads();
    if (threadIdx.x == 0) {
      st->status = ST_DONE;
      st->path = PATH_EXACT;
      st->count = 0;
      st->r_sampled = 0;
      st->tau_key = 0;
      st->ties = 0;
      st->tau_route = TAU_NONE;
      st->passes = 0;
    }
  };
  if (small_k && k <= RF_RANK_MAX && n <= ER_STREAM_MAX) {
    uint32_t* s_hist2048 = reinterpret_cast<uint32_t*>(s_cand + CAND_CAP / 2);
    const bool done =
        n <= 8 * blockDim.x
            ? exact_row_in_registers<DT, 8>(rowp, n, k, B, out_values, out_idx, row, s_hist,
                                            s_misc, s_hist2048, s_cand)
            : exact_row_streamed<DT>(values, n, k, B, out_values, out_idx, row, s_hist, s_misc,
                                     s_hist2048, s_cand);
    if (done) {
      finish_row();
      return;
    }
    __syncthreads();   // every thread has read the bin search's result
  }
  RowSrc<DT> src{rowp, B, (1ull << B) - 1ull};
  SelectOut sel = block_select(src, n, W, k, k, s_hist, s_misc, s_cand, CAND_CAP);
  if (small_k) {
    const uint32_t got = block_collect(src, n, sel.thr, s_cand, CAND_CAP, &s_misc[4]);
    const uint32_t P = next_pow2(got);
    for (uint32_t i = got + threadIdx.x; i < P; i += blockDim.x) s_cand[i] = 0ull;
    __syncthreads();
    block_bitonic_desc(s_cand, P);
    write_winners<DT>(s_cand, k, k, B, rowp, n, out_values, out_idx, row);
    finish_row();
    return;
  }
  // large k: scatter the k winners to global memory
  uint64_t* out = cbuf + (size_t)row * cap;
  if (threadIdx.x == 0) {
    s_misc[4] = 0;
    s_misc[5] = 0;
  }
  __syncthreads();
  uint32_t km = 0;   // largest winner key
  for (uint32_t i0 = 0; i0 < n; i0 += blockDim.x) {
    const uint32_t i = i0 + threadIdx.x;
    uint64_t c = 0;
    bool keep = false;
    if (i < n) {
      c = src(i);
      keep = c >= sel.thr;
    }
    if (keep && (uint32_t)(c >> B) > km) km = (uint32_t)(c >> B);
    const uint64_t m = ballot(keep);
    if (m) {
      const uint32_t first = (uint32_t)__builtin_ctzll(m);
      uint32_t base = 0;
      if (lane_id() == first) base = atomicAdd(&s_misc[4], (uint32_t)__builtin_popcountll(m));
      base = wave_bcast(base, first);
      const uint32_t slot = base + rank_below(m);
      if (keep && slot < cap) out[slot] = c;
    }
  }
  km = wave_max_u32(km);
  if (lane_id() == 0 && km) atomicMax(&s_misc[5], km);
  __syncthreads();
  if (threadIdx.x == 0) {
    st->count = s_misc[4] < cap ? s_misc[4] : cap;
    st->thr_key = (uint32_t)(sel.thr >> B);   // every winner key is >= this
    st->kmax = s_misc[5];
    st->status = ST_SORT;
    st->path = PATH_EXACT;
    st->r_sampled = 0;
    st->tau_key = 0;
    st->ties = 0;
    st->tau_route = TAU_NONE;
    st->passes = 0;
  }
}
