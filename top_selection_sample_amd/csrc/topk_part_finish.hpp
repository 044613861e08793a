// Exact route helpers, the bucket-sort digit, and the finish kernel (k_finish).
// A part of topk_kernels.hip, included there in order inside namespace tk;
// it relies on the definitions of the parts before it and is not a
// stand-alone header.
#pragma once

// ======================================================================
// Exact route (Prof-K section 3, stage 4: exact top-k on the full input when
// the sampled filter fails), done as a radix select over each listed row:
// every pass counts one 8-bit digit of the composite over the elements that
// match the resolved prefix; a workgroup per row then resolves the boundary
// bucket.  Passes stop as soon as the elements at or above the bucket fit the
// candidate buffer, so the scratch memory stays O(capacity), never O(n).
// Then one filter pass with the exact threshold fills the buffer, and the
// rows are refined (small k) or handed to the sort (large k).
//
// One launch does it all, the phases separated by grid-wide barriers.  The
// grid is one workgroup per compute unit, so all workgroups are normally
// resident together.  Every barrier wait is bounded: a workgroup whose wait
// gives up (not every workgroup is resident: other work holds compute units)
// sets CallState::error and leaves the shared phases, which makes every
// later barrier give up as well, so no phase ever runs on another
// workgroup's unfinished data.  The last workgroup to finish (an exit
// ticket) then selects every listed row again by itself, exactly: slow, but
// the answer stays the exact top-k.  The same launch first refines the rows
// whose sampled candidates passed the check, so when no row failed the exact
// route costs nothing beyond that launch.
// ======================================================================

// Arrival: a release fence (this workgroup's writes reach memory), then one
// relaxed increment of the arrival count; the last arrival acquires the
// others' writes, resets the count and bumps the generation.  Waiting polls
// the generation with relaxed loads and acquires once it has moved: an
// acquiring load per poll would invalidate the L2 at every iteration, which
// measured about four times slower on MI355X (~22 us against ~6 us per
// barrier over 256 workgroups).  Returns false (the same in every thread)
// when the wait gave up after `spin_limit` polls.  s_flag: one LDS word.
__device__ bool grid_barrier(CallState* cs, uint32_t G, uint32_t spin_limit, uint32_t* s_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t ok = 1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t gen = __hip_atomic_load(&cs->bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t arrived =
        __hip_atomic_fetch_add(&cs->bar_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    if (arrived == G) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(&cs->bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&cs->bar_gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t spins = 0;
      while (__hip_atomic_load(&cs->bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        if (spins >= spin_limit) {
          __hip_atomic_fetch_or(&cs->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        ++spins;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  return ok;
}

constexpr uint32_t EX_THREADS = 1024;
static_assert(EX_THREADS == RS_THREADS, "k_finish runs refine_sampled with its workgroup");
static_assert(RF_RANK_MAX * 4 <= EX_THREADS, "rank counting: four lanes per element");
constexpr uint32_t EX_VPT = 4;                            // vectors per thread per item
constexpr uint32_t EX_ITEM_VEC = EX_THREADS * EX_VPT;     // vectors per item

// (match, digit) of one element for the pass that resolves bits
// [W - nb - 8, W - nb) of the composite key << B | (2^B - 1 - idx).
template <int KBITS>
__device__ __forceinline__ bool digit_of(uint32_t key, uint32_t idx, uint32_t nb, uint64_t prefix,
                                         uint32_t B, uint32_t* d) {
  if (nb < (uint32_t)KBITS) {                 // a key digit
    const uint32_t pkey = (uint32_t)(prefix >> B);
    const bool m = (nb == 0) || ((key >> (KBITS - nb)) == (pkey >> (KBITS - nb)));
    *d = (key >> (KBITS - nb - 8)) & 255u;
    return m;
  }
  const uint32_t ib = nb - KBITS;             // resolved index bits
  const uint32_t low = (uint32_t)(((1ull << B) - 1ull) - idx);
  const uint32_t plow = (uint32_t)(prefix & ((1ull << B) - 1ull));
  const bool m = (key == (uint32_t)(prefix >> B)) && (ib == 0 || (low >> (B - ib)) == (plow >> (B - ib)));
  *d = (low >> (B - ib - 8)) & 255u;
  return m;
}

struct RowGeom {
  const char* rowp;
  uint32_t head, nvec, tail0;
  const u32x4* vp;
};

template <int DT>
__device__ __forceinline__ RowGeom row_geom(const void* values, uint32_t n, uint32_t row) {
  using D = Dt<DT>;
  RowGeom g;
  g.rowp = static_cast<const char*>(values) + (size_t)row * n * D::ES;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(g.rowp);
  g.head = (uint32_t)(((16u - (addr & 15u)) & 15u) / D::ES);
  if (g.head > n) g.head = n;
  g.nvec = (n - g.head) / D::VEC;
  g.tail0 = g.head + g.nvec * D::VEC;
  g.vp = reinterpret_cast<const u32x4*>(g.rowp + (size_t)g.head * D::ES);
  return g;
}

// ======================================================================
// Large k, capacity up to LK_CAP_MAX: bucket sort of the candidates.
// Composites are unique and every candidate key lies in [lo, kmax] (lo =
// RowState::thr_key, the threshold the candidates passed; kmax tracked by
// the filters), so
//     v = (key - lo) << bl | (low bl bits of the inverted index)
// (bl = index bits that vary, 2^bl >= n) orders the candidates exactly as
// their composites do, with no constant bits in between.  Its top 12 bits
// are the bucket, and its rank r = 4095 - bucket (ranks ascend as buckets
// descend, so the output is the buckets in rank order):
//   chunk step    (lk_sort_chunk: in k_finish, in k_lk_chunk for rows that
//                 never pass through it) per 4096 candidates: the chunk
//                 rewritten in place grouped by rank, with its prefix count
//                 per rank (LDS counting sort; no global atomics)
//   k_lk_sort     one workgroup per LK_WIN output positions: the bucket
//                 start of rank r is the sum over the chunks of their prefix
//                 counts at r; a search over r finds the ranks whose buckets
//                 start in the window, their candidates are gathered from
//                 every chunk (each chunk holds them as one run), sorted in
//                 LDS and written as winners; a bucket too large for LDS is
//                 split further in the workgroup (11-bit digits below the
//                 common prefix of its smallest and largest value, through
//                 the split scratch).
// A global bucket histogram built with atomics measured about 10 us slower
// to read back in the next kernel (2^28 bf16, k = 131072: 166k atomics on
// 4096 words) than data written with plain stores, however its words were
// spread over lines or channels; the sums over the chunks avoid it.
// Workspace: lkc (u32) [rows][chunks][4096] the chunks' prefix counts by
// rank; lks (u64) [rows][cap] the split scratch.
// ======================================================================
constexpr uint32_t LK_BITS = 12;
constexpr uint32_t LK_BINS = 1u << LK_BITS;
static_assert(LK_BINS == LK_RANKS && LK_CSTRIDE == LK_BINS + 64,
              "per chunk: LK_BINS prefix counts, then every 64th of them");
constexpr uint32_t LK_THREADS = 1024;
constexpr uint32_t LK_CHUNK = 4 * LK_THREADS;   // candidates per chunk step
constexpr uint32_t LK_WIN = 1024;               // output positions per sort workgroup
constexpr uint32_t LK_LCAP = 2048;              // largest range sorted in LDS
constexpr uint32_t LK_STACK = 1024;             // pending oversized ranges per workgroup
constexpr uint32_t LK_MAXCH = (uint32_t)(LK_CAP_MAX / LK_CHUNK);   // chunks of a row at most
static_assert((int64_t)LK_STACK * LK_LCAP >= LK_CAP_MAX,
              "oversized ranges are disjoint and larger than LK_LCAP, so at most "
              "LK_CAP_MAX / LK_LCAP of them are ever pending");
static_assert(LK_LCAP >= 2 * LK_WIN, "a window's small buckets fit one LDS sort");

// Chunks of LK_CHUNK candidates in a row's buffer of capacity cap.
__device__ __forceinline__ uint32_t lk_maxch(uint32_t cap) { return (cap + LK_CHUNK - 1) / LK_CHUNK; }
static_assert(LK_BINS == 4 * LK_THREADS && LK_CHUNK == 4 * LK_THREADS && LK_CHUNK == LK_CHUNK_CANDS,
              "a chunk step: four candidates and four ranks per thread");

struct LkDigit {
  uint32_t B, bl, lo, shift;
  uint64_t low;
  // v of a composite, and back
  __device__ uint64_t compact(uint64_t c) const { return (((c >> B) - lo) << bl) | (c & low); }
  __device__ uint64_t expand(uint64_t v) const {
    const uint64_t mask_b = (B >= 64) ? ~0ull : ((1ull << B) - 1ull);
    return (((v >> bl) + lo) << B) | (mask_b & ~low) | (v & low);
  }
  __device__ uint32_t operator()(uint64_t c) const {   // bucket of a composite
    const uint64_t d = compact(c) >> shift;
    return d < LK_BINS ? (uint32_t)d : LK_BINS - 1;   // (always below: key <= kmax)
  }
};

__device__ __forceinline__ LkDigit lk_digit(uint32_t lo, uint32_t kmax, uint32_t B, uint32_t bl) {
  LkDigit g;
  g.B = B;
  g.bl = bl;
  g.lo = lo;
  g.low = (1ull << bl) - 1ull;   // bl <= 32
  const uint32_t hi = kmax > g.lo ? kmax : g.lo;
  const uint64_t vmax = ((uint64_t)(hi - g.lo) << bl) | g.low;
  const uint32_t tb = vmax ? 64u - (uint32_t)__builtin_clzll(vmax) : 0u;
  g.shift = tb > LK_BITS ? tb - LK_BITS : 0u;
  return g;
}

__device__ __forceinline__ LkDigit lk_digit_of(const RowState& st, uint32_t B, uint32_t bl) {
  return lk_digit(st.thr_key, st.kmax, B, bl);
}

// One LK_CHUNK of a row's candidates, [base, base + len) with len =
// min(LK_CHUNK, R - base): an LDS histogram of its buckets, then the chunk
// written back to out[base, base + len) grouped by rank (rank r = LK_BINS -
// 1 - bucket: ranks ascend as buckets descend), with pre[r] = the number of
// the chunk's candidates of ranks below r (LK_BINS words) and pre[LK_BINS +
// m] = pre[64 m] (64 words, for the window search).  Candidate i is cb[i] below G and tb[i - G] from G on (the tie
// region, for a sampled row whose ties were never copied over).  out may be
// cb: the workgroup reads its chunk before it writes it, and no other
// workgroup touches [base, base + len).  Every thread of the workgroup
// (LK_CHUNK / 4 of them) calls it; h: LK_BINS + 16 words of LDS, s_sorted:
// LK_CHUNK composites of LDS.
__device__ void lk_sort_chunk(const uint64_t* __restrict__ cb, const uint64_t* __restrict__ tb,
                              uint32_t G, uint32_t R, uint32_t base, const LkDigit& g,
                              uint64_t* out, uint32_t* __restrict__ pre, uint32_t* h,
                              uint64_t* s_sorted) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x, lane = tid & 63u, w = tid >> 6;
  uint32_t* s_wsum = h + LK_BINS;
  for (uint32_t i = tid; i < LK_BINS; i += nt) h[i] = 0;
  uint64_t c[4];
  uint32_t bk[4];
  bool ok[4];
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t i = base + j * nt + tid;
    ok[j] = i < R;
    c[j] = ok[j] ? (i < G ? cb[i] : tb[i - G]) : 0ull;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    bk[j] = ok[j] ? g(c[j]) : 0u;
    hist_add(h, bk[j], ok[j]);
  }
  __syncthreads();
  // ranks 4 tid .. 4 tid + 3: their exclusive prefix in rank order
  uint32_t hv[4], sum = 0;
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    hv[j] = h[LK_BINS - 1 - (4 * tid + j)];
    sum += hv[j];
  }
  const uint32_t incl = wave_incl_sum(sum);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();   // (also: every count read before the counts become cursors)
  uint32_t run = incl - sum;
  for (uint32_t i = 0; i < nt / 64; ++i) run += i < w ? s_wsum[i] : 0u;
  if ((tid & 15u) == 0) pre[LK_BINS + (tid >> 4)] = run;   // rank 4 tid = 64 (tid / 16)
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    pre[4 * tid + j] = run;
    h[LK_BINS - 1 - (4 * tid + j)] = run;
    run += hv[j];
  }
  __syncthreads();
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j)
    if (ok[j]) s_sorted[atomicAdd(&h[bk[j]], 1u)] = c[j];
  __syncthreads();
  const uint32_t len = R - base < LK_CHUNK ? R - base : LK_CHUNK;
  for (uint32_t i = tid; i < len; i += nt) out[base + i] = s_sorted[i];
  __syncthreads();
}

// How the finish kernel learns which rows failed the check.
//  FIN_SCAN: sampled route with at most FIN_SCAN_ROWS rows: every workgroup
//    reads every row's survivor count itself.  All reach the same verdict
//    without waiting for one another: a count is final once the filter has
//    run, and the only write to it here (start_exact, on a failed row) keeps
//    the row failed.  The common case (no failure) then needs no barrier.
//  FIN_LISTED: an earlier kernel listed the failed rows (nflag, flagged[]).
enum : uint32_t { FIN_SCAN = 0, FIN_LISTED = 1 };
// k_finish runs the bucket sort's chunk step for the accepted sampled rows
// and/or for the exact route's rows (large k).
enum : uint32_t { LK_HIST_SAMPLED = 1, LK_HIST_EXACT = 2, FIN_SMALL_K = 4 };
constexpr uint32_t FIN_SCAN_ROWS = 1024;

// One listed row selected again by one workgroup (every thread calls it):
// the exact route's work for that row with no other workgroup involved, used
// when a grid-barrier wait gave up.  A radix select of the k-th composite
// over the whole row, then (small k) its k winners sorted in LDS and written,
// or (large k) the k winners into the row's candidate buffer, its bucket
// histogram rebuilt and the row handed to the sort.  LDS as in k_finish.
template <int DT>
__device__ __attribute__((noinline)) void reselect_row(const void* __restrict__ values, uint32_t n, RowState* st,
                             uint32_t row, uint64_t* __restrict__ cbuf, uint32_t cap, uint32_t k,
                             uint32_t B, uint32_t W, uint32_t small_k,
                             void* __restrict__ out_values, int64_t* __restrict__ out_idx,
                             uint32_t* __restrict__ pre_row, uint32_t bl, uint32_t* s_hist,
                             uint32_t* s_misc, uint64_t* s_cand, uint32_t* s_keys) {
  using D = Dt<DT>;
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * D::ES;
  const RowSrc<DT> src{rowp, B, (1ull << B) - 1ull};
  // passes stop once exactly k composites lie at or above the bucket
  const SelectOut sel = block_select(src, n, W, k, k, s_hist, s_misc, s_cand, RF_SORT_CAP);
  if (small_k) {   // k <= KSMALL = RF_SORT_CAP
    const uint32_t got = block_collect(src, n, sel.thr, s_cand, RF_SORT_CAP, &s_misc[4]);
    const uint32_t P = next_pow2(got);
    for (uint32_t i = got + tid; i < P; i += nt) s_cand[i] = 0ull;
    __syncthreads();
    block_bitonic_desc(s_cand, P);
    write_winners<DT>(s_cand, k, k, B, rowp, n, out_values, out_idx, row);
    __syncthreads();
    if (tid == 0) st->status = ST_DONE;
    __syncthreads();
    return;
  }
  uint64_t* out = cbuf + (size_t)row * cap;
  if (tid == 0) {
    s_misc[4] = 0;
    s_misc[5] = 0;
  }
  __syncthreads();
  uint32_t km = 0;
  for (uint32_t i0 = 0; i0 < n; i0 += nt) {
    const uint32_t i = i0 + tid;
    const uint64_t c = i < n ? src(i) : 0ull;
    const bool keep = i < n && c >= sel.thr;
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
  const uint32_t R = s_misc[4] < cap ? s_misc[4] : cap;
  const uint32_t thr_key = (uint32_t)(sel.thr >> B), kmax = s_misc[5];
  if (pre_row) {   // the chunks grouped by rank, for the bucket sort
    const LkDigit g = lk_digit(thr_key, kmax, B, bl);
    for (uint32_t base = 0; base < R; base += LK_CHUNK)
      lk_sort_chunk(out, out, R, R, base, g, out, pre_row + (size_t)(base / LK_CHUNK) * LK_CSTRIDE,
                    s_keys, s_cand);
  }
  if (tid == 0) {
    st->count = R;
    st->thr_key = thr_key;   // every winner key is >= this
    st->kmax = kmax;
    st->status = ST_SORT;
  }
  __syncthreads();
}

// The exact route of k_finish (every row that failed the check, nf > 0 in
// every workgroup): a function of its own, called only then, so that its
// registers do not crowd those of the common path (check and refine).  The
// LDS arrays are k_finish's.
template <int DT>
__device__ __attribute__((noinline)) void finish_exact(
    const void* __restrict__ values, uint32_t n, uint32_t rows, RowState* __restrict__ states,
    CallState* __restrict__ cs, uint32_t* __restrict__ flagged, uint32_t* __restrict__ ghist,
    uint64_t* __restrict__ cbuf, uint32_t cap, uint32_t k, uint32_t B, uint32_t W,
    uint32_t small_k, uint32_t mode, void* __restrict__ out_values, int64_t* __restrict__ out_idx,
    uint32_t* __restrict__ lkc, uint32_t bl, uint32_t lk_flags, uint32_t spin_limit, uint32_t G,
    uint32_t nf, uint32_t* s_hist, uint32_t* s_misc, uint32_t* s_tmp, uint64_t* s_cand,
    uint32_t* s_keys, uint32_t* s_idx, uint32_t* s_flag_p) {
  using D = Dt<DT>;
  const uint32_t tid = threadIdx.x, w = tid >> 6;
  uint32_t& s_flag = *s_flag_p;
  // ======================= exact route (nf > 0 in every workgroup) =======
  // A listed entry always names a row of this call once the barrier after
  // the listing has passed; the bound is kept anyway for every read.
  auto listed = [&](uint32_t f) -> uint32_t {
    const uint32_t r = flagged[f];
    return r < rows ? r : 0xFFFFFFFFu;
  };
  if (mode == FIN_SCAN && blockIdx.x == 0 && tid == 0) {
    cs->nflag = nf;
    cs->nactive = nf;
  }
  // per-call scratch: the listed rows' exact-route histograms start at zero
  for (uint32_t f = blockIdx.x; f < nf; f += G)
    if (tid < 256) ghist[(size_t)f * 256 + tid] = 0u;
  bool ok = grid_barrier(cs, G, spin_limit, &s_flag);   // the listed rows' states are visible to all

  uint32_t ipr = (n / D::VEC + EX_ITEM_VEC - 1) / EX_ITEM_VEC;   // items per row
  if (ipr == 0) ipr = 1;
  const uint64_t total = (uint64_t)nf * ipr;

  // Listed row f covers items [f * ipr, (f + 1) * ipr).  Each workgroup takes
  // one contiguous range of items, so it streams long runs of one row and
  // reads a row's state only when the row changes.
  const uint64_t per = (total + G - 1) / G;
  const uint64_t it_lo = (uint64_t)blockIdx.x * per;
  const uint64_t it_hi = it_lo + per < total ? it_lo + per : total;
  constexpr uint32_t SPAN = EX_VPT * D::VEC;   // elements per thread per item
  const uint32_t lane = tid & 63u;
  auto vec_of = [&](uint32_t c, uint32_t b) { return c * EX_ITEM_VEC + (b / D::VEC) * EX_THREADS + tid; };
  auto load_item = [&](const RowGeom& g, uint32_t c, u32x4 (&xs)[EX_VPT]) {
#pragma unroll
    for (uint32_t j = 0; j < EX_VPT; ++j) {
      const uint32_t v = c * EX_ITEM_VEC + j * EX_THREADS + tid;
      xs[j] = v < g.nvec ? __builtin_nontemporal_load(g.vp + v) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // The elements before the first and after the last 16-byte vector of a
  // row (fewer than 2 * VEC): visited with item 0 by the first wave.
  auto head_tail = [&](const RowGeom& g, auto&& f) {
    if (tid < 64) {
      const uint32_t nt = n - g.tail0;
      const bool ok = tid < g.head + nt;
      uint32_t idx = 0, raw = 0;
      if (ok) {
        idx = (tid < g.head) ? tid : g.tail0 + (tid - g.head);
        raw = load_raw<DT>(g.rowp, idx);
      }
      f(raw, idx, ok);
    }
  };

  // ---- histogram passes
  for (uint32_t pass = 0; ok && pass < W / 8; ++pass) {
    if (__hip_atomic_load(&cs->nactive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) break;
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();
    uint32_t fcur = 0xFFFFFFFFu, nb = 0;
    uint64_t prefix = 0;
    bool live = false;
    RowGeom g{};
    // the LDS histogram collects consecutive items of one row
    auto flush_hist = [&]() {
      __syncthreads();
      if (tid < 256) {
        const uint32_t h = s_hist[tid];
        if (h) {
          atomicAdd(&ghist[(size_t)fcur * 256 + tid], h);
          s_hist[tid] = 0;
        }
      }
      __syncthreads();
    };
    for (uint64_t it = it_lo; it < it_hi; ++it) {
      const uint32_t f = (uint32_t)(it / ipr), c = (uint32_t)(it % ipr);
      if (f != fcur) {
        if (live) flush_hist();
        fcur = f;
        const uint32_t row = listed(f);
        live = row != 0xFFFFFFFFu && states[row].status == ST_EXACT;
        if (live) {
          const RowState* st = states + row;
          nb = st->nbits;
          prefix = st->prefix;
          g = row_geom<DT>(values, n, row);
        }
      }
      if (!live) continue;
      u32x4 xs[EX_VPT];
      load_item(g, c, xs);
      // Count this thread's matching elements and whether they share one
      // digit; when the whole wave does (skewed data, late passes) one atomic
      // adds the wave's count, else every element adds itself.
      uint32_t my_d = 0, my_cnt = 0;
      bool uni = true;
#pragma unroll
      for (uint32_t b = 0; b < SPAN; ++b) {
        uint32_t d;
        const uint32_t e = g.head + vec_of(c, b) * D::VEC + b % D::VEC;
        const bool act = vec_of(c, b) < g.nvec &&
                         digit_of<D::KB>(D::key(elemvc<DT, EX_VPT>(xs, b)), e, nb, prefix, B, &d);
        if (act) {
          uni = uni && (my_cnt == 0 || d == my_d);
          my_d = my_cnt == 0 ? d : my_d;
          ++my_cnt;
        }
      }
      const uint64_t has = ballot(my_cnt != 0u);
      if (has) {
        const uint32_t dref = wave_bcast(my_d, (uint32_t)__builtin_ctzll(has));
        const bool agree = my_cnt == 0u || (uni && my_d == dref);
        if (ballot(!agree) == 0) {
          uint32_t tcount = my_cnt;
          tcount = wave_sum_u32(tcount);
          if (lane == 0) atomicAdd(&s_hist[dref], tcount);
        } else {
#pragma unroll
          for (uint32_t b = 0; b < SPAN; ++b) {
            uint32_t d;
            const uint32_t e = g.head + vec_of(c, b) * D::VEC + b % D::VEC;
            const bool act = vec_of(c, b) < g.nvec &&
                             digit_of<D::KB>(D::key(elemvc<DT, EX_VPT>(xs, b)), e, nb, prefix, B, &d);
            if (act) atomicAdd(&s_hist[d], 1u);
          }
        }
      }
      if (c == 0) {
        head_tail(g, [&](uint32_t raw, uint32_t idx, bool ok) {
          uint32_t d;
          const bool m = digit_of<D::KB>(D::key(raw), idx, nb, prefix, B, &d);
          hist_add(s_hist, d, ok && m);
        });
      }
    }
    if (live) flush_hist();
    ok = grid_barrier(cs, G, spin_limit, &s_flag);
    if (!ok) break;
    // resolve: one workgroup per listed row
    for (uint32_t f = blockIdx.x; f < nf; f += G) {
      const uint32_t row = listed(f);
      if (row == 0xFFFFFFFFu) continue;
      RowState* st = states + row;
      if (st->status != ST_EXACT) continue;
      uint32_t* gh = ghist + (size_t)f * 256;
      if (tid < 256) {
        s_hist[tid] = gh[tid];
        gh[tid] = 0;
      }
      __syncthreads();
      const uint32_t need = st->need;
      if (tid < 64) wave_find_bucket(s_hist, need, s_misc);
      __syncthreads();
      if (tid == 0) {
        const uint32_t nb0 = st->nbits;
        const uint32_t shift = W - nb0 - 8;
        const uint32_t b = s_misc[0], acc = s_misc[1], hb = s_misc[2];
        const uint32_t above = st->above + acc;
        const uint64_t np = st->prefix | ((uint64_t)b << shift);
        const uint32_t nnb = nb0 + 8;
        const uint64_t maskB = (1ull << B) - 1ull;
        st->above = above;
        st->need = need - acc;
        st->prefix = np;
        st->nbits = nnb;
        st->passes = st->passes + 1;
        if (above + hb <= cap || nnb >= W) {
          st->thr_key = (uint32_t)(np >> B);
          st->thr_bound = (uint32_t)(maskB - (np & maskB));
          st->count = 0;
          st->kmax = 0;
          st->status = ST_EXACT_READY;
          atomicSub(&cs->nactive, 1u);
        }
      }
      __syncthreads();
    }
    ok = grid_barrier(cs, G, spin_limit, &s_flag);
  }

  // ---- exact filter: every element >= the exact threshold into the buffer
  if (ok) {
    Stager sg{s_cand + (size_t)w * STAGE_SLOTS, 0u, nullptr, nullptr, cap, nullptr, B, 0u};
    const uint64_t maskB = (1ull << B) - 1ull;
    auto comp = [&](uint32_t raw, uint32_t idx) -> uint64_t {
      return ((uint64_t)D::key(raw) << B) | (maskB - idx);
    };
    uint32_t fcur = 0xFFFFFFFFu;
    bool live = false;
    Thr thr{};
    RowGeom g{};
    for (uint64_t it = it_lo; it < it_hi; ++it) {
      const uint32_t f = (uint32_t)(it / ipr), c = (uint32_t)(it % ipr);
      if (f != fcur) {
        if (sg.fill) sg.flush();   // to the previous row
        sg.publish();
        fcur = f;
        const uint32_t row = listed(f);
        live = row != 0xFFFFFFFFu && states[row].status == ST_EXACT_READY;
        if (live) {
          RowState* st = states + row;
          thr = make_thr<DT>(st->thr_key, st->thr_bound);
          sg.ctr = &st->count;
          sg.kmax = &st->kmax;
          sg.buf = cbuf + (size_t)row * cap;
          g = row_geom<DT>(values, n, row);
        }
      }
      if (!live) continue;
      u32x4 xs[EX_VPT];
      load_item(g, c, xs);
      uint32_t bits = 0;
#pragma unroll
      for (uint32_t b = 0; b < SPAN; ++b) {
        const uint32_t e = g.head + vec_of(c, b) * D::VEC + b % D::VEC;
        const bool p = vec_of(c, b) < g.nvec && key_pass(D::key(elemvc<DT, EX_VPT>(xs, b)), e, thr);
        bits |= (uint32_t)p << b;
      }
      drain_bits<DT, EX_VPT>(
          sg, xs, bits,
          [&](uint32_t b) { return g.head + vec_of(c, b) * D::VEC + b % D::VEC; }, comp);
      if (c == 0) {
        head_tail(g, [&](uint32_t raw, uint32_t idx, bool ok) {
          const bool p = ok && key_pass(D::key(raw), idx, thr);
          sg.push(p, p ? comp(raw, idx) : 0ull);
        });
      }
    }
    if (sg.fill) sg.flush();
    sg.publish();
    ok = grid_barrier(cs, G, spin_limit, &s_flag);
  }

  // ---- refine (small k) or hand over to the sort (large k)
  if (ok) {
    for (uint32_t f = blockIdx.x; f < nf; f += G) {
      const uint32_t row = listed(f);
      if (row == 0xFFFFFFFFu) continue;
      if (small_k) {
        refine_row<DT>(values, n, states, cs, flagged, cbuf, cap, k, B, W, ST_EXACT_READY,
                       out_values, out_idx, row, s_hist, s_misc, s_tmp, s_cand, s_keys, s_idx);
      } else if (tid == 0) {
        states[row].status = ST_SORT;
      }
    }
    // Large k: the chunk step for the exact route's rows (their count,
    // threshold and largest key were final at the last grid barrier)
    if (!small_k && (lk_flags & LK_HIST_EXACT)) {
      const uint32_t maxch = lk_maxch(cap);
      const uint64_t npairs = (uint64_t)nf * maxch;
      for (uint64_t q = blockIdx.x; q < npairs; q += G) {
        const uint32_t row = listed((uint32_t)(q / maxch)), c = (uint32_t)(q % maxch);
        if (row == 0xFFFFFFFFu) continue;
        const RowState st = states[row];
        const uint32_t R = st.count < cap ? st.count : cap;
        if ((uint64_t)c * LK_CHUNK >= R) continue;
        lk_sort_chunk(cbuf + (size_t)row * cap, cbuf + (size_t)row * cap, R, R, c * LK_CHUNK,
                      lk_digit_of(st, B, bl), cbuf + (size_t)row * cap,
                      lkc + ((size_t)row * maxch + c) * LK_CSTRIDE, s_keys, s_cand);
      }
    }
  }

  // ---- exit ticket.  Every workgroup takes one after its last write; the
  // last one sees every other workgroup's writes.  If any barrier wait gave
  // up, it selects every listed row again on its own.
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t t =
        __hip_atomic_fetch_add(&cs->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = t == G - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_flag = last && (__hip_atomic_load(&cs->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1u);
  }
  __syncthreads();
  if (!s_flag) return;
  for (uint32_t f = 0; f < nf; ++f) {
    const uint32_t row = listed(f);
    if (row == 0xFFFFFFFFu) continue;
    reselect_row<DT>(values, n, states + row, row, cbuf, cap, k, B, W, small_k, out_values,
                     out_idx,
                     (lk_flags & LK_HIST_EXACT) ? lkc + (size_t)row * lk_maxch(cap) * LK_CSTRIDE
                                                : nullptr,
                     bl, s_hist, s_misc, s_cand, s_keys);
  }
}

template <int DT>
// flags: FIN_SMALL_K | LK_HIST_SAMPLED | LK_HIST_EXACT.  The arguments the
// check and the refine need come first (the first 14 words of the argument
// block arrive in scalar registers with the launch); G = the grid size,
// passed rather than read from the dispatch's hidden arguments; the
// composite width W = B + the key bits; the call record, the flagged-row
// list and the exact-route histograms sit at offsets that follow from rows.
__global__ __launch_bounds__(EX_THREADS) void k_finish(
    RowState* __restrict__ states, const RowCtr* __restrict__ rctr, uint64_t* __restrict__ cbuf,
    uint32_t rows, uint32_t mode, uint32_t k, uint32_t k_eff, uint32_t cap, uint32_t flags,
    uint32_t B, uint32_t G, const void* __restrict__ values, uint32_t n,
    const uint64_t* __restrict__ tbuf, void* __restrict__ out_values,
    int64_t* __restrict__ out_idx, uint32_t* __restrict__ lkc, uint32_t bl,
    uint32_t spin_limit) {
  using D = Dt<DT>;
  assume_block_threads(EX_THREADS);
  const uint32_t W = B + D::KB;
  CallState* __restrict__ cs = ws_region<CallState>(states, ws_off_call(rows));
  uint32_t* __restrict__ flagged = ws_region<uint32_t>(states, ws_off_flag(rows));
  uint32_t* __restrict__ ghist = ws_region<uint32_t>(states, ws_off_ghist(rows));
  const uint32_t small_k = (flags & FIN_SMALL_K) ? 1u : 0u;
  const uint32_t lk_flags = flags & (LK_HIST_SAMPLED | LK_HIST_EXACT);
  __shared__ __align__(16) uint32_t s_hist[RF_BINS];
  __shared__ uint32_t s_misc[8];
  __shared__ uint32_t s_tmp[16];
  __shared__ uint64_t s_cand[RF_SORT_CAP];
  __shared__ uint32_t s_keys[RF_KCAP];
  __shared__ uint32_t s_idx[RF_SORT_CAP];
  __shared__ uint32_t s_flag;
  const uint32_t tid = threadIdx.x, w = tid >> 6;

  // FIN_SCAN (a sampled call): this workgroup's first row's state is read
  // here, in the same round trip as the check's reads below (as vector
  // loads, which go out together: the compiler serialises scalar loads here
  // to save scalar registers)
  const uint32_t r_first = blockIdx.x;
  const bool pre = mode == FIN_SCAN && r_first < rows;
  uint32_t f_status = 0, f_count = 0, f_ties = 0, f_kmax = 0, f_tau = 0;
  if (pre) {
    auto ld = [](const uint32_t* q) {
      return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    f_status = ld(&states[r_first].status);
    f_count = ld(&rctr[r_first].above);
    f_tau = ld(&states[r_first].tau_key);
    f_ties = ld(&rctr[r_first].ties);
    f_kmax = ld(&rctr[r_first].kmax);
  }
  static_assert(FIN_SCAN_ROWS % 32 == 0, "whole words of row bits");

  // ---- which rows failed the check (Prof-K section 3, stage 4).  Every
  // count read here is final and never rewritten in this kernel (the
  // filter's above-tau count and tie count), so every workgroup reaches the
  // same verdict for every row.
  __shared__ uint32_t s_bad[FIN_SCAN_ROWS / 32];   // FIN_SCAN: one bit per row
  uint32_t nf;
  if (mode == FIN_SCAN) {
    // (rows <= FIN_SCAN_ROWS = the workgroup: one row per thread; both
    // counts are read before the LDS set-up, unconditionally at a clamped
    // row, so the two loads go out together)
    static_assert(FIN_SCAN_ROWS <= EX_THREADS, "one row per thread");
    const uint32_t words = (rows + 31) / 32;
    const uint32_t rr = tid < rows ? tid : rows - 1;
    const uint32_t Ga = __hip_atomic_load(&rctr[rr].above, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t Ea = __hip_atomic_load(&rctr[rr].ties, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (uint32_t i = tid; i < words; i += blockDim.x) s_bad[i] = 0u;
    __syncthreads();
    if (tid < rows && sampled_verdict(Ga, Ea, k, k_eff, cap) == V_FAIL)
      atomicOr(&s_bad[tid >> 5], 1u << (tid & 31));
    __syncthreads();
    nf = 0;
    for (uint32_t i = 0; i < words; ++i) nf += __builtin_popcount(s_bad[i]);
  } else {
    nf = __hip_atomic_load(&cs->nflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (nf > rows) nf = rows;   // (at most one entry per row was listed)
  }

  // ---- this workgroup's rows: list the failed ones, refine the others
  for (uint32_t r = blockIdx.x; r < rows; r += G) {
    RowState* st = states + r;
    if (mode == FIN_SCAN && nf && (s_bad[r >> 5] >> (r & 31)) & 1u) {
      if (tid == 0) {
        uint32_t slot = 0;   // failed rows below r
        for (uint32_t i = 0; i < (r >> 5); ++i) slot += __builtin_popcount(s_bad[i]);
        slot += __builtin_popcount(s_bad[r >> 5] & ((1u << (r & 31)) - 1u));
        st->ties = rctr[r].ties;
        st->r_sampled = rctr[r].above + st->ties;
        start_exact(st, k, PATH_FALLBACK);
        flagged[slot] = r;
      }
      // (large k: the chunk step below skips failed rows)
      continue;
    }
    const bool fr = pre && r == r_first;
    if ((fr ? f_status : st->status) != ST_FILTER) continue;
    // an accepted row; when it needs the ties, they join its candidates
    const uint32_t G = fr ? f_count : rctr[r].above, E = fr ? f_ties : rctr[r].ties;
    const uint32_t kmx = fr ? f_kmax : rctr[r].kmax, tau = fr ? f_tau : st->tau_key;
    const uint32_t verdict = sampled_verdict(G, E, k, k_eff, cap);
    const bool ties_in = verdict == V_OK_TIES || verdict == V_PARTIAL;
    if (!fr) __syncthreads();   // every thread has read the counts
    // (the bucket sort's chunk step reads them from the tie region instead)
    const bool copy_ties = ties_in && !(lk_flags & LK_HIST_SAMPLED);
    if (copy_ties) {
      uint64_t* dst = cbuf + (size_t)r * cap + G;
      const uint64_t* src = tbuf + (size_t)r * cap;
      for (uint32_t i = tid; i < E; i += blockDim.x) dst[i] = src[i];
    }
    if (tid == 0) {
      st->r_sampled = G + E;
      st->ties = E;
      if (G < k) st->count = G + E;
      if (verdict == V_PARTIAL) st->path = PATH_PARTIAL;
      if (!small_k) {
        st->thr_key = st->tau_key;   // every candidate key is >= this
        st->kmax = rctr[r].kmax;
        st->status = ST_SORT;
      }
    }
    if (copy_ties) __syncthreads();   // the copied ties are visible to every thread
    if (small_k) {
      uint32_t R = G < k ? G + E : G;
      if (R > cap) R = cap;
      // a partial row (fewer than k reach tau) keeps all R and pads the rest
      const uint32_t kk = R < k ? R : k;
      refine_sampled<DT>(values, n, st, cbuf + (size_t)r * cap, R, tau, kmx, kk, k, B, W,
                         out_values, out_idx, r, s_hist, s_misc, s_tmp, s_cand,
                         reinterpret_cast<uint64_t*>(s_keys));
    }
  }
  // Large k: the bucket histograms of the accepted sampled rows and their
  // chunks grouped by rank (the first step of the bucket sort), LK_CHUNK
  // candidates per workgroup and step.  Every count read here is final: the
  // filter's above-tau count and tie count, tau and the largest key (the
  // row's owner rewrites only the RowState count).  A row's ties are read
  // from the tie region: for large k they are never copied into the
  // candidate buffer, whose chunks are rewritten here.
  if (lk_flags & LK_HIST_SAMPLED) {
    const uint32_t maxch = lk_maxch(cap);
    const uint64_t npairs = (uint64_t)rows * maxch;
    for (uint64_t q = blockIdx.x; q < npairs; q += G) {
      const uint32_t r = (uint32_t)(q / maxch), c = (uint32_t)(q % maxch);
      const uint32_t Ga = rctr[r].above, E = rctr[r].ties;
      const uint32_t v = sampled_verdict(Ga, E, k, k_eff, cap);
      if (v == V_FAIL) continue;   // the exact route's rows: below
      uint32_t R = (v == V_OK_TIES || v == V_PARTIAL) ? Ga + E : Ga;
      if (R > cap) R = cap;
      if ((uint64_t)c * LK_CHUNK >= R) continue;
      const LkDigit g = lk_digit(states[r].tau_key, rctr[r].kmax, B, bl);
      lk_sort_chunk(cbuf + (size_t)r * cap, tbuf + (size_t)r * cap, Ga, R, c * LK_CHUNK, g,
                    cbuf + (size_t)r * cap, lkc + ((size_t)r * maxch + c) * LK_CSTRIDE, s_keys,
                    s_cand);
    }
  }
  if (nf == 0) return;                        // the common case: nothing more to do
  finish_exact<DT>(values, n, rows, states, cs, flagged, ghist, cbuf, cap, k, B, W, small_k, mode,
                   out_values, out_idx, lkc, bl, lk_flags, spin_limit, G, nf, s_hist, s_misc,
                   s_tmp, s_cand, s_keys, s_idx, &s_flag);
}
