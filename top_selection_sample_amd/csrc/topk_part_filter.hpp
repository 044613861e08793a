// Filter, detection and exact-route setup kernels (k_filter, k_check, k_setup_exact).
// A part of topk_kernels.hip, included there in order inside namespace tk;
// it relies on the definitions of the parts before it and is not a
// stand-alone header.
#pragma once

// ======================================================================
// Filter (Prof-K section 3, stage 3; Appendix D "Efficient GPU
// Implementation"): one streaming pass over the row that keeps every element
// whose key is >= the threshold.  The survivors are split in two: those
// strictly above tau are appended to the row's candidate buffer, those equal
// to tau are counted exactly and stored in a tie region of the same capacity
// while it has room.  When at least k survivors lie strictly above tau the
// ties cannot be among the answer, so ties alone never make a row overflow;
// otherwise the row needs all of them (see sampled_verdict).  The counters
// keep counting past the capacity; a wave that meets a full above-tau buffer
// stops early (the row overflows, so only "more than the capacity" matters).
//
// Survivor slots come from a wave ballot and the count of set lanes below
// each lane (the stable split's count of earlier elements with the same
// flag, GPU.js Learn "One Bit at a Time"); they are staged per wave in LDS and each
// workgroup appends its survivors with one atomic at the end.
// ======================================================================
// Launch shape (measured on MI355X): 512-thread workgroups, one per compute
// unit (two when survivors are dense), each streaming one contiguous slice
// of its row with four 16-byte nontemporal loads per lane and the next four
// issued before the current ones are examined; long per-workgroup streams
// beat a grid-stride sweep by about 20%.
constexpr uint32_t FILTER_THREADS = 512;
constexpr uint32_t FILTER_WAVES = FILTER_THREADS / 64;
constexpr uint32_t STAGE_SLOTS = 128;
constexpr uint32_t FILTER_UNROLL = 4;
// hit-queue entries per wave: fewer than 64 wait between steps, and one
// step adds at most FILTER_UNROLL * 64
constexpr uint32_t HITQ = 64 * (FILTER_UNROLL + 1);

struct Stager {
  uint64_t* stage;   // this wave's LDS slots
  uint32_t fill;     // wave-uniform
  uint32_t* ctr;     // the buffer's slot counter
  uint64_t* buf;     // the buffer
  uint32_t cap;
  uint32_t* kmax;    // if set: publish() raises it to the largest key stored
  uint32_t kshift;   //   (key = comp >> kshift)
  uint32_t km;       // wave-uniform: largest key flushed since the last publish
  uint32_t flushed = 0;   // wave-uniform: entries counted by flush() so far

  // Returns true when the buffer is full.
  __device__ bool flush() {
    wave_lds_sync();
    uint32_t base = 0;
    if (lane_id() == 0) base = atomicAdd(ctr, fill);
    base = wave_bcast(base, 0u);
    uint32_t m = 0;
    for (uint32_t i = lane_id(); i < fill; i += 64) {
      const uint32_t pos = base + i;
      if (pos < cap) buf[pos] = stage[i];
      const uint32_t key = (uint32_t)(stage[i] >> kshift);
      m = key > m ? key : m;
    }
    if (kmax) {
      m = wave_max_u32(m);
      km = m > km ? m : km;
    }
    wave_lds_sync();
    const bool full = base + fill > cap;
    flushed += fill;
    fill = 0;
    return full;
  }
  // One wave's largest key into *kmax (a read first: most waves find it
  // already larger and skip the contended atomic).
  __device__ void publish() {
    if (kmax && km && lane_id() == 0 &&
        km > __hip_atomic_load(kmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(kmax, km);
    km = 0;
  }
  // All lanes call together.
  __device__ void push(bool p, uint64_t comp) {
    const uint64_t m = ballot(p);
    if (!m) return;
    const uint32_t c = (uint32_t)__builtin_popcountll(m);
    if (fill + c > STAGE_SLOTS) flush();
    if (p) stage[fill + rank_below(m)] = comp;
    fill += c;
  }
};

// Element b (0 .. NV * VEC - 1) of NV 16-byte vectors as raw bits; b may
// differ between lanes (a select chain, no indexed register access).
template <int DT, int NV>
__device__ __forceinline__ uint32_t elemv(const u32x4 (&v)[NV], uint32_t b) {
  using D = Dt<DT>;
  const uint32_t u = b / D::VEC, e = b % D::VEC;
  u32x4 w = v[0];
#pragma unroll
  for (int j = 1; j < NV; ++j) w = (u == (uint32_t)j) ? v[j] : w;
  if constexpr (DT == DT_BF16) {
    const uint32_t q = e >> 1;
    const uint32_t x = q == 0 ? w[0] : q == 1 ? w[1] : q == 2 ? w[2] : w[3];
    return (e & 1u) ? (x >> 16) : (x & 0xFFFFu);
  } else {
    return e == 0 ? w[0] : e == 1 ? w[1] : e == 2 ? w[2] : w[3];
  }
}

// The same with b known at compile time (unrolled loops).
template <int DT, int NV>
__device__ __forceinline__ uint32_t elemvc(const u32x4 (&v)[NV], uint32_t b) {
  using D = Dt<DT>;
  const uint32_t u = b / D::VEC, e = b % D::VEC;
  if constexpr (DT == DT_BF16) return (e & 1u) ? (v[u][e >> 1] >> 16) : (v[u][e >> 1] & 0xFFFFu);
  else return v[u][e];
}

// Survivors of one step: each lane holds one bit per passing element; the
// wave drains the bits one survivor per lane per round (slot = set lanes
// below, as in push), so a lane with one survivor costs one round whatever
// the element's position.  idx_of(b) is the index of element b, comp_of
// builds its composite.  All lanes call together; returns true when a flush
// found the buffer full.
template <int DT, int NV, class IdxF, class CompF>
__device__ __forceinline__ bool drain_bits(Stager& sg, const u32x4 (&v)[NV], uint32_t bits,
                                           IdxF&& idx_of, CompF&& comp_of) {
  bool full = false;
  uint64_t m = ballot(bits != 0u);
  while (m) {
    const uint32_t c = (uint32_t)__builtin_popcountll(m);
    if (sg.fill + c > STAGE_SLOTS) full = sg.flush() || full;
    if (bits) {
      const uint32_t b = (uint32_t)__builtin_ctz(bits);
      bits &= bits - 1u;
      sg.stage[sg.fill + rank_below(m)] = comp_of(elemv<DT, NV>(v, b), idx_of(b));
    }
    sg.fill += c;
    m = ballot(bits != 0u);
  }
  return full;
}

// The same drain with the survivors split on the way: is_tie(raw) sends an
// element to the tie stager tg (while the tie region is not full) and counts
// it, every other survivor goes to sg.  For sparse survivors, where a
// per-survivor test is cheaper than a second mask over every element.
struct SplitOut {
  bool full;       // sg found its buffer full
  bool tfull;      // the tie region is full
  uint32_t ties;   // this lane's ties drained
};

template <int DT, int NV, class IdxF, class CompF, class TieF>
__device__ __forceinline__ SplitOut drain_split(Stager& sg, Stager& tg, bool tfull,
                                                const u32x4 (&v)[NV], uint32_t bits,
                                                IdxF&& idx_of, CompF&& comp_of, TieF&& is_tie) {
  bool full = false;
  uint32_t ties = 0;
  uint64_t m = ballot(bits != 0u);
  while (m) {
    const bool has = bits != 0u;
    uint32_t b = 0, raw = 0;
    bool e = false;
    if (has) {
      b = (uint32_t)__builtin_ctz(bits);
      bits &= bits - 1u;
      raw = elemv<DT, NV>(v, b);
      e = is_tie(raw);
    }
    ties += e ? 1u : 0u;
    const uint64_t mg = ballot(has && !e), me = ballot(e);
    if (mg) {
      const uint32_t c = (uint32_t)__builtin_popcountll(mg);
      if (sg.fill + c > STAGE_SLOTS) full = sg.flush() || full;
      if (has && !e) sg.stage[sg.fill + rank_below(mg)] = comp_of(raw, idx_of(b));
      sg.fill += c;
    }
    if (me && !tfull) {
      const uint32_t c = (uint32_t)__builtin_popcountll(me);
      if (tg.fill + c > STAGE_SLOTS) tfull = tg.flush();
      if (!tfull) {
        if (e) tg.stage[tg.fill + rank_below(me)] = comp_of(raw, idx_of(b));
        tg.fill += c;
      }
    }
    m = ballot(bits != 0u);
  }
  return SplitOut{full, tfull, ties};
}

// Native-domain threshold for the fast compare.  kind 0: compare in the value
// domain; kind 1: compare keys (thresholds above +inf, or a tie cut on index).
struct Thr {
  float f;
  int32_t i;
  uint32_t key;
  uint32_t bound;
  int kind;
};

template <int DT>
__device__ __forceinline__ Thr make_thr(uint32_t key, uint32_t bound) {
  Thr t;
  t.key = key;
  t.bound = bound;
  t.kind = (bound != 0xFFFFFFFFu) ? 1 : 0;
  t.i = (int32_t)(key ^ 0x80000000u);
  t.f = 0.f;
  if constexpr (DT == DT_F32) {
    if (key > 0xFF800000u) t.kind = 1;                       // only NaN passes
    else if (key <= 0x007FFFFFu) t.f = -__builtin_huge_valf();  // everything passes
    else t.f = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
  } else if constexpr (DT == DT_BF16) {
    if (key > 0xFF80u) t.kind = 1;
    else if (key <= 0x007Fu) t.f = -__builtin_huge_valf();
    else {
      const uint32_t b16 = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
      t.f = __uint_as_float(b16 << 16);
    }
  }
  return t;
}

// key >= thr, with the index cut on the threshold key.
__device__ __forceinline__ bool key_pass(uint32_t key, uint32_t idx, const Thr& t) {
  return key > t.key || (key == t.key && idx <= t.bound);
}

template <int DT>
__device__ __forceinline__ bool native_pass(uint32_t raw, const Thr& t) {
  if constexpr (DT == DT_I32) return (int32_t)raw >= t.i;
  else if constexpr (DT == DT_F32) return !(__uint_as_float(raw) < t.f);
  else return !(__uint_as_float(raw << 16) < t.f);
}

// Equal to the threshold value (+0 and -0 are equal, NaN equals nothing).
template <int DT>
__device__ __forceinline__ bool native_eq(uint32_t raw, const Thr& t) {
  if constexpr (DT == DT_I32) return (int32_t)raw == t.i;
  else if constexpr (DT == DT_F32) return __uint_as_float(raw) == t.f;
  else return __uint_as_float(raw << 16) == t.f;
}

// bf16 screen of a 16-byte vector (eight elements) for the plain-threshold
// loop: whether some element's magnitude bits reach tau's bits, with packed
// 16-bit operations (a mask of the sign bits, three maxima, one saturating
// subtraction), where the exact test takes two instructions per element and
// a scalar OR per pair.  With tau > 0 (tb1x2 = tau's bits - 1 in both halves)
// every passing element is caught: a positive one at or above tau, and NaN
// of either sign, whose magnitude bits exceed every finite value's.  The
// screen also flags negative elements of magnitude >= tau; the survivor code
// tests each flagged element exactly, so that only costs a queue entry.  With
// tau <= 0 (all = true) every vector is flagged: most elements pass then.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bool bf16_screen(const u32x4& v, uint32_t tb1x2, bool all) {
  auto mag = [](uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu); };
  const u16x2 a = __builtin_elementwise_max(mag(v[0]), mag(v[1]));
  const u16x2 b = __builtin_elementwise_max(mag(v[2]), mag(v[3]));
  const u16x2 d = __builtin_elementwise_sub_sat(__builtin_elementwise_max(a, b),
                                                __builtin_bit_cast(u16x2, tb1x2));
  return all || __builtin_bit_cast(uint32_t, d) != 0u;
}

// tau from the sampler's per-workgroup top-t lists (ns keys, list g at
// [g t, g t + t), largest first), by one filter workgroup, for ns up to
// FILTER_THREADS * TL_PER keys and any t <= TOPT; thread tid holds key
// q * FILTER_THREADS + tid in v[q] (values at or past ns are ignored).
// (Inlined, so that it runs while the first loads of the stream are in
// flight.)  tau is at least lo, the
// largest list tail (the t-th largest of one workgroup's sample), and at
// most hi, the largest head; the keys >= lo share the bits above the top
// differing bit of lo and hi, so a radix select with 11-bit digits below
// that prefix, over the keys held in registers, resolves it in one level
// when lo and hi differ only in their low 11 bits (else two or three).
// s_hist: 2048 words; s_red: 2 * FILTER_WAVES + 4 words.  Every thread calls it.
constexpr uint32_t TL_PER = 8;   // list keys per thread
__device__ __forceinline__ uint32_t tau_from_lists(const uint32_t (&v)[TL_PER], uint32_t ns, uint32_t t,
                                                   uint32_t* s_hist, uint32_t* s_red) {
  const uint32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63u;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (uint32_t q = 0; q < TL_PER; ++q) {
    const uint32_t i = q * FILTER_THREADS + tid;
    const bool ok = i < ns;
    const uint32_t r = i % t;
    if (ok && r == 0) hi = v[q] > hi ? v[q] : hi;
    if (ok && r == t - 1) lo = v[q] > lo ? v[q] : lo;
  }
  lo = wave_max_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    s_red[w] = lo;
    s_red[FILTER_WAVES + w] = hi;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t j = 0; j < FILTER_WAVES; ++j) {   // independent reads
    const uint32_t a = s_red[j], b = s_red[FILTER_WAVES + j];
    lo = a > lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  uint32_t diff = lo ^ hi;
  if (diff == 0) return lo;   // every key >= lo equals lo: the t-th largest is lo
  // resolved: the bits above `pos`, equal to those of pfx (the prefix of lo
  // and hi to start with); need: the rank wanted among the keys matching it
  uint32_t pos = 32u - (uint32_t)__builtin_clz(diff);   // bits below the common prefix
  uint32_t pfx = lo & ~((pos >= 32u) ? 0xFFFFFFFFu : ((1u << pos) - 1u));
  uint32_t need = t;
  while (pos > 0) {
    const uint32_t width = pos < 11u ? pos : 11u;
    const uint32_t shift = pos - width;
    const uint32_t hmask = (pos >= 32u) ? 0u : ~((1u << pos) - 1u);   // the resolved bits
    for (uint32_t i = tid; i < 2048; i += FILTER_THREADS) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (uint32_t q = 0; q < TL_PER; ++q) {
      const bool act = q * FILTER_THREADS + tid < ns && v[q] >= lo && (v[q] & hmask) == pfx;
      hist_add(s_hist, (v[q] >> shift) & ((1u << width) - 1u), act);
    }
    __syncthreads();
    if (tid < 64) wave_find_bucket_2048(s_hist, need, s_red + 2 * FILTER_WAVES);
    __syncthreads();
    const uint32_t b = s_red[2 * FILTER_WAVES], acc = s_red[2 * FILTER_WAVES + 1];
    __syncthreads();
    need -= acc;
    pfx |= b << shift;
    pos = shift;
  }
  return pfx;
}

// tau from the sampler's sorted per-workgroup lists of TOPT = 32 keys (list
// g at keys [32 g, 32 g + 32), largest first), for 8 < t <= 32 and ns <=
// FILTER_THREADS * TL_PER keys: the t-th largest of their union, by bitonic
// merges that keep the 32 largest.  Thread tid holds key q * FILTER_THREADS
// + tid in v[q] (keys at or past ns count as 0, which cannot raise the t-th
// largest), so each register of a wave holds two whole lists, one per half:
// the second reversed makes the 64 lanes bitonic and one merge leaves the
// pair's 32 largest, sorted, in lanes 0-31.  The eight registers are merged
// pairwise in three more rounds, then one wave merges the eight waves'
// lists.  s_m: FILTER_WAVES * 32 + 1 words.  Every thread calls it.
__device__ __forceinline__ uint32_t tau_from_sorted32(const uint32_t (&v0)[TL_PER], uint32_t ns,
                                                      uint32_t t, uint32_t* s_m) {
  static_assert(TOPT == 32 && FILTER_THREADS % 64 == 0, "two lists of 32 per wave register");
  const uint32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63u;
  // (only the registers that hold keys: the merges are VALU-bound, and with
  // two workgroups per compute unit sixteen waves share its four SIMDs)
  const uint32_t nq = (ns + FILTER_THREADS - 1) / FILTER_THREADS;   // 1 .. TL_PER, uniform
  uint32_t v[TL_PER];
#pragma unroll
  for (uint32_t q = 0; q < TL_PER; ++q) {
    v[q] = 0u;
    if (q < nq) {
      const uint32_t x = q * FILTER_THREADS + tid < ns ? v0[q] : 0u;
      const uint32_t y = (uint32_t)__shfl((int)x, (int)(lane < 32 ? lane : 95u - lane), 64);
      v[q] = wave_merge_desc(y);
    }
  }
  auto pair = [&](uint32_t a, uint32_t b) {   // lanes 0-31 of a, then lanes 31..0 of b
    const uint32_t rb = (uint32_t)__shfl((int)b, (int)(63u - lane), 64);
    return wave_merge_desc(lane < 32 ? a : rb);
  };
#pragma unroll
  for (uint32_t step = 1; step < TL_PER; step <<= 1) {
#pragma unroll
    for (uint32_t q = 0; q + step < TL_PER; q += 2 * step)
      if (q + step < nq) v[q] = pair(v[q], v[q + step]);
  }
  if (lane < 32) s_m[w * 32 + lane] = v[0];
  __syncthreads();
  if (w == 0) {
    uint32_t x[FILTER_WAVES];
#pragma unroll
    for (uint32_t j = 0; j < FILTER_WAVES; ++j) x[j] = s_m[j * 32 + (lane & 31u)];
#pragma unroll
    for (uint32_t step = 1; step < FILTER_WAVES; step <<= 1) {
#pragma unroll
      for (uint32_t j = 0; j + step < FILTER_WAVES; j += 2 * step) x[j] = pair(x[j], x[j + step]);
    }
    if (lane == t - 1) s_m[FILTER_WAVES * 32] = x[0];
  }
  __syncthreads();
  return s_m[FILTER_WAVES * 32];
}

// The filter's body.  AHEAD3: three steps of the stream are loaded before tau
// is known instead of two (for the merge of sorted lists, whose tau comes
// last: on 2^28 bf16 with t = 32 0.6 us less per call; with an early tau the
// extra registers cost more than they save).
// The arguments the prologue needs come first: the first 14 words of the
// argument block arrive in scalar registers with the launch, the rest takes a
// memory round trip.  bpr = the grid's x size (workgroups per row), passed
// rather than read from the dispatch's hidden arguments for the same reason.
#define TK_FILTER_PARAMS                                                                      \
  const void* __restrict__ values, const uint32_t* __restrict__ tlist,                        \
      RowState* __restrict__ states, uint32_t n, uint32_t tlist_n, uint32_t tlist_stride,     \
      uint32_t t, uint32_t bpr, uint32_t cap, uint32_t B, uint32_t track_kmax,                \
      RowCtr* __restrict__ rctr, uint64_t* __restrict__ cbuf, uint64_t* __restrict__ tbuf,    \
      WsHeader* validate, uint64_t sig, uint64_t* __restrict__ wg_trace, uint32_t trace_wgs
#define TK_FILTER_ARGS                                                                        \
  values, tlist, states, n, tlist_n, tlist_stride, t, bpr, cap, B, track_kmax, rctr, cbuf,    \
      tbuf, validate, sig, wg_trace, trace_wgs
template <int DT, bool AHEAD3>
__device__ __forceinline__ void filter_body(TK_FILTER_PARAMS) {
  using D = Dt<DT>;
  assume_block_threads(FILTER_THREADS);
  const uint32_t row = blockIdx.y;
  RowState* st = states + row;
  Thr thr;   // set below, once tau is known
  // (measurement aid: realtime stamps of this workgroup's start and the end
  // of its scan)
  const uint32_t lwg = row * bpr + blockIdx.x;
  const bool traced = wg_trace && lwg < trace_wgs;
  if (traced && threadIdx.x == 0) wg_trace[2 * (size_t)lwg] = __builtin_amdgcn_s_memrealtime();

  __shared__ __align__(16) uint64_t s_stage[FILTER_WAVES][STAGE_SLOTS];   // (16: the prologue bins)
  __shared__ uint64_t s_tstage[FILTER_WAVES][STAGE_SLOTS];
  __shared__ uint32_t s_fill[FILTER_WAVES], s_tfill[FILTER_WAVES], s_ties[FILTER_WAVES],
      s_flushed[FILTER_WAVES];
  __shared__ uint32_t s_base, s_tbase, s_km;
  const uint32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63u;
  if (tid == 0) s_km = 0;
  RowCtr* rc = rctr + row;
  // above tau (and, for large k, its largest key: the bucket sort's range)
  Stager sg{s_stage[w], 0u, &st->count, cbuf + (size_t)row * cap, cap, nullptr, B, 0u};
  Stager tg{s_tstage[w], 0u, &rc->tslots, tbuf + (size_t)row * cap, cap, nullptr, B, 0u};  // = tau
  if (track_kmax) sg.kmax = &rc->kmax;

  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * D::ES;
  const uint64_t maskB = (1ull << B) - 1ull;
  auto comp_of = [&](uint32_t raw, uint32_t idx) -> uint64_t {
    return ((uint64_t)D::key(raw) << B) | (maskB - idx);
  };
  auto pass_of = [&](uint32_t raw) -> bool {
    if (thr.kind == 0) return native_pass<DT>(raw, thr);
    return D::key(raw) >= thr.key;
  };
  auto eq_of = [&](uint32_t raw) -> bool {
    if (thr.kind == 0) return native_eq<DT>(raw, thr);
    return D::key(raw) == thr.key;
  };

  // Split the row into an unaligned head, 16-byte vectors, and a tail.
  const uintptr_t addr = reinterpret_cast<uintptr_t>(rowp);
  uint32_t head = (uint32_t)(((16u - (addr & 15u)) & 15u) / D::ES);
  if (head > n) head = n;
  const uint32_t nvec = (n - head) / D::VEC;
  const uint32_t tail0 = head + nvec * D::VEC;
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + (size_t)head * D::ES);

  uint32_t ties = 0;      // this lane's elements equal to tau
  bool full = false;      // the above-tau buffer is full: the row overflows
  bool tfull = false;     // the tie region is full: ties are only counted

  // One element outside the unrolled loop (all lanes call together).
  auto push_one = [&](bool p, uint32_t raw, uint32_t idx) {
    const bool e = p && eq_of(raw);
    ties += e ? 1u : 0u;
    const uint64_t c = p ? comp_of(raw, idx) : 0ull;
    sg.push(p && !e, c);
    if (!tfull) tg.push(e, c);
  };

  // Survivors of one 16-byte vector (VEC elements per lane, a bit each),
  // drained by drain_split or drain_bits.  A wave that finds the above-tau
  // buffer full stops scanning: the row overflows and goes to the exact route
  // whatever the rest would count.  A full tie region only stops the storing
  // of ties.  Per vector rather than per unrolled step: with many survivors
  // (bf16 at large k: most 2048-element steps hold one) the masks and drains
  // then cover 8 elements instead of 32.
  auto vec_survivors = [&](const u32x4& v0, size_t vi_lane, bool ok) __attribute__((always_inline)) {
    const u32x4 v[1] = {v0};
    auto idx_of = [&](uint32_t b) { return head + (uint32_t)vi_lane * D::VEC + b; };
    uint32_t ge = 0;
#pragma unroll
    for (uint32_t b = 0; b < D::VEC; ++b) ge |= (uint32_t)pass_of(elemvc<DT, 1>(v, b)) << b;
    if (!ok) ge = 0u;
    if (ballot(__builtin_popcount(ge) > D::VEC / 2) == 0) {
      // sparse survivors: test each one for a tie as it is drained
      const SplitOut o = drain_split<DT, 1>(sg, tg, tfull, v, ge, idx_of, comp_of, eq_of);
      full = full || o.full;
      tfull = o.tfull;
      ties += o.ties;
      return;
    }
    // dense (many ties, or a threshold below most of the row): a tie mask.
    // The empty asm on the copy keeps these compares inside this rare
    // branch; otherwise the compiler computes them for every vector of the
    // hot loop.
    u32x4 w[1] = {v0};
    asm volatile("" : "+v"(w[0]));
    uint32_t eq = 0;
#pragma unroll
    for (uint32_t b = 0; b < D::VEC; ++b) eq |= (uint32_t)eq_of(elemvc<DT, 1>(w, b)) << b;
    eq &= ge;
    ties += (uint32_t)__builtin_popcount(eq);
    full = drain_bits<DT, 1>(sg, v, ge & ~eq, idx_of, comp_of) || full;
    if (!tfull && ballot(eq != 0u)) tfull = drain_bits<DT, 1>(tg, v, eq, idx_of, comp_of);
  };

  // The hit queue of the plain-threshold loop: a lane whose vector holds a
  // survivor appends the vector and its index to its wave's LDS ring; after
  // a step, while 64 or more are queued, the wave examines 64 of them
  // together, one per lane.  With sparse survivors (a lane in a few hundred)
  // the drains then run with every lane busy instead of one, at the cost of
  // one LDS write per hit.  (One place drains, so the drain code is inlined
  // once: as a call, the loop's state would live in scratch memory, whose
  // loads wait for every load in flight.)
  __shared__ u32x4 s_qv[FILTER_WAVES][HITQ];
  __shared__ uint32_t s_qi[FILTER_WAVES][HITQ];
  uint32_t q_head = 0, q_cnt = 0;   // wave-uniform; q_cnt < 64 between steps
  auto wrapq = [](uint32_t e) { return e >= HITQ ? e - HITQ : e; };   // e < 2 HITQ
  // (DENSE: the counting mode, whose ties were counted in the compare loop:
  // only the elements above tau are stored)
  auto drain_queue_t = [&](uint32_t cnt, auto dense_tag) __attribute__((always_inline)) {
    wave_lds_sync();
    const bool ok = lane < cnt;
    const uint32_t e = wrapq(q_head + lane);
    const u32x4 x = ok ? s_qv[w][e] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t xi = ok ? s_qi[w][e] : 0u;
    q_head = wrapq(q_head + cnt);
    q_cnt -= cnt;
    if constexpr (decltype(dense_tag)::value) {
      const u32x4 v[1] = {x};
      uint32_t gt = 0;
#pragma unroll
      for (uint32_t b = 0; b < D::VEC; ++b) {
        const uint32_t y = elemvc<DT, 1>(v, b);
        gt |= (uint32_t)(pass_of(y) && !eq_of(y)) << b;
      }
      if (!ok) gt = 0u;
      full = drain_bits<DT, 1>(
                 sg, v, gt, [&](uint32_t b) { return head + xi * D::VEC + b; }, comp_of) ||
             full;
    } else {
      vec_survivors(x, xi, ok);
    }
  };
  auto drain_queue = [&](uint32_t cnt) __attribute__((always_inline)) {
    drain_queue_t(cnt, std::false_type{});
  };
  auto drain_queue_dense = [&](uint32_t cnt) __attribute__((always_inline)) {
    drain_queue_t(cnt, std::true_type{});
  };
  auto enqueue = [&](bool hit, uint64_t hm, const u32x4& x, uint32_t xi) {
    if (hit) {
      const uint32_t e = wrapq(q_head + q_cnt + rank_below(hm));
      s_qv[w][e] = x;
      s_qi[w][e] = xi;
    }
    q_cnt += (uint32_t)__builtin_popcountll(hm);
  };

  // This workgroup's slice of the row's vectors: [vi0, vend), in steps of
  // FILTER_THREADS * FILTER_UNROLL vectors.
  constexpr size_t step = (size_t)FILTER_THREADS * FILTER_UNROLL;
  const size_t per = (((size_t)nvec + bpr - 1) / bpr + step - 1) / step * step;
  const size_t vi0 = (size_t)blockIdx.x * per;
  const size_t vend = vi0 + per < (size_t)nvec ? vi0 + per : (size_t)nvec;
  constexpr size_t stride = FILTER_THREADS;
  size_t vi = vi0 + tid;
  // Main loop: FILTER_UNROLL independent 16-byte nontemporal loads per lane.
  // The bound is tested on the wave's last lane, so every lane of a wave runs
  // the same trip count (the ballots and the staging counter need that).
  // With a plain threshold the loop only ORs native compares and skips the
  // vectors of a wave that has no survivor.
  // The loads of the next step are issued before the current step is
  // examined, so a wave that is draining survivors still has a step's worth
  // of loads in flight.  The first two steps' loads go out before tau is
  // known, so that selecting it overlaps more of the stream.
  // (the same for every lane of the wave; said so with readfirstlane, so that
  // the loads below sit behind scalar branches: behind lane-masked ones the
  // loaded registers are merged with their old values, and the merge copy
  // waits for the loads)
  auto step_ok = [&](size_t at) {
    const bool ok = (at - lane) + 63 + (FILTER_UNROLL - 1) * stride < vend;
    return __builtin_amdgcn_readfirstlane(ok ? 1 : 0) != 0;
  };
  // tau's inputs are read first: loads complete in order, so a wait for
  // them must not come after the stream's first loads
  uint32_t tlv[TL_PER];
  {
    const uint32_t* kl = tlist_n ? tlist + (size_t)row * tlist_stride
                                 : reinterpret_cast<const uint32_t*>(st);
    const uint32_t klast = tlist_n ? tlist_n - 1 : 0u;
#pragma unroll
    for (uint32_t q = 0; q < TL_PER; ++q) {
      const uint32_t i = q * FILTER_THREADS + tid;
      tlv[q] = kl[i < klast ? i : klast];   // (clamped: masked where used)
    }
  }
  // so are the row's state and, when k_tau or the caller set it, tau: read
  // after the stream's first loads, they came back only after them (about
  // 2 us with one workgroup per unit, 4 with two)
  const uint32_t row_status = st->status;
  const uint32_t tau_given = tlist_n ? 0u : st->tau_key;
  constexpr size_t sstep = FILTER_UNROLL * stride;
  u32x4 nxt[FILTER_UNROLL], nx2[FILTER_UNROLL], nx3[FILTER_UNROLL];
  const bool more2_ = step_ok(vi + sstep);
  const bool more3_ = step_ok(vi + 2 * sstep);
  bool more = step_ok(vi);
  bool more2 = more && more2_;
  {
    // unconditional, at clamped indices (a step that is not taken loads
    // vectors it never reads; with no vectors at all, the row state): no
    // branch, so nothing merges these registers and waits for the loads
    const u32x4* vq = nvec ? vp : reinterpret_cast<const u32x4*>(st);
    const size_t vlast = nvec ? (size_t)nvec - 1 : 0;
#pragma unroll
    for (uint32_t u = 0; u < FILTER_UNROLL; ++u) {
      const size_t i0 = vi + u * stride, i1 = i0 + sstep, i2 = i1 + sstep;
      nxt[u] = __builtin_nontemporal_load(vq + (i0 < vlast ? i0 : vlast));
      nx2[u] = __builtin_nontemporal_load(vq + (i1 < vlast ? i1 : vlast));
      if constexpr (AHEAD3) nx3[u] = __builtin_nontemporal_load(vq + (i2 < vlast ? i2 : vlast));
    }
  }
  // (after the loads above: a row left to another route reads and discards
  // them, and stores nothing; the empty asm keeps the compiler from moving
  // this check, and its wait for the row state, in front of them)
  asm volatile("" ::: "memory");
  if (row_status != ST_FILTER) return;
  // k_tau has left every row's sample histogram zero: stamp the workspace
  if (validate && row == 0 && blockIdx.x == 0 && tid == 0) validate->stamp = sig;
  // tau: given by k_tau, or (tlist_n > 0) the t-th largest of the sampler's
  // per-workgroup top-t lists, selected here by every workgroup
  uint32_t tau;
  if (tlist_n) {
    __shared__ uint32_t s_tl[FILTER_WAVES * 8], s_tc[2 * FILTER_WAVES + 4], s_to[8];
    if (t <= 8 && tlist_n <= 4 * FILTER_THREADS) {
      // few small lists: the t largest by wave max extraction
      uint32_t v[4], cnt = 0;
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) {
        const bool ok = q * FILTER_THREADS + tid < tlist_n;
        v[q] = ok ? tlv[q] : 0u;
        cnt += ok ? 1u : 0u;
      }
      block_top_t4<FILTER_WAVES, 8>(v, cnt, t, s_tl, s_tc, s_to);
      tau = s_to[t - 1];   // the lists hold at least t keys
    } else if (t > TOPT_EXTRACT) {
      // (sorted lists of 32; the staging area is free until the loop)
      tau = tau_from_sorted32(tlv, tlist_n, t, reinterpret_cast<uint32_t*>(&s_stage[0][0]));
    } else {
      // (the staging area is free until the loop: its first 8 KB hold the bins)
      tau = tau_from_lists(tlv, tlist_n, t, reinterpret_cast<uint32_t*>(&s_stage[0][0]), s_tc);
    }
    if (blockIdx.x == 0 && tid == 0) st->tau_key = tau;
  } else {
    tau = tau_given;
  }
  thr = make_thr<DT>(tau, 0xFFFFFFFFu);
  // (bf16: the screen's constant, and whether it flags every vector)
  const bool scr_all = !(thr.f > 0.f);
  const uint32_t scr_tb1 = scr_all ? 0u : ((__float_as_uint(thr.f) >> 16) - 1u) * 0x10001u;
  if (thr.kind == 0) {
    // one step: the compares, the hits queued, then the drains the queue
    // calls for (all that is left after the last step)
    auto scan_step = [&](const u32x4 (&v)[FILTER_UNROLL], size_t vc, bool last)
                         __attribute__((always_inline)) {
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) {
        uint32_t any = 0;
        if constexpr (DT == DT_BF16) {
          any = bf16_screen(v[u], scr_tb1, scr_all) ? 1u : 0u;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) any |= (uint32_t)native_pass<DT>(v[u][q], thr);
        }
        const uint64_t hm = ballot(any != 0u);
        if (hm) enqueue(any != 0u, hm, v[u], (uint32_t)(vc + u * stride));
      }
      while (q_cnt >= 64u || (last && q_cnt)) drain_queue(q_cnt < 64u ? q_cnt : 64u);
    };
    // the same in the counting mode: ties counted as they are compared, and
    // only vectors with an element above tau queued
    auto scan_step_dense = [&](const u32x4 (&v)[FILTER_UNROLL], size_t vc, bool last)
                               __attribute__((always_inline)) {
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) {
        uint32_t gt = 0, eqn = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          auto one = [&](uint32_t x) {
            const bool eq = native_eq<DT>(x, thr);
            gt |= (uint32_t)(native_pass<DT>(x, thr) && !eq);
            eqn += eq ? 1u : 0u;
          };
          if constexpr (DT == DT_BF16) {
            one(v[u][q] & 0xFFFFu);
            one(v[u][q] >> 16);
          } else {
            one(v[u][q]);
          }
        }
        ties += eqn;
        const uint64_t hm = ballot(gt != 0u);
        if (hm) enqueue(gt != 0u, hm, v[u], (uint32_t)(vc + u * stride));
      }
      while (q_cnt >= 64u || (last && q_cnt)) drain_queue_dense(q_cnt < 64u ? q_cnt : 64u);
    };
    // The first step straight from its registers, the second one's loads
    // still in flight; from then on one step ahead (the registers of the
    // next step are copied into those of the current one, and a copy waits
    // for its loads).
    if (more) {
      const size_t vc = vi;
      vi += sstep;
      scan_step(nxt, vc, !more2);
      more = more2 && !full;
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) nxt[u] = nx2[u];
    }
    // (AHEAD3) the second step, the third one's loads still in flight (with the tie
    // region full, the counting loop takes the second step and loads the
    // third again)
    if (AHEAD3 && more && !tfull) {
      const size_t vc = vi;
      vi += sstep;
      scan_step(nxt, vc, !more3_);
      more = more3_ && !full;
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) nxt[u] = nx3[u];
    }
    while (more && !tfull) {   // (the tie region full: on to the counting loop)
      u32x4 v[FILTER_UNROLL];
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) v[u] = nxt[u];
      const size_t vc = vi;
      vi += sstep;
      more = step_ok(vi);
      if (more) {
#pragma unroll
        for (uint32_t u = 0; u < FILTER_UNROLL; ++u)
          nxt[u] = __builtin_nontemporal_load(vp + vi + u * stride);
      }
      scan_step(v, vc, !more);
      if (full) break;
    }
    // the tie region is full (and the queue empty): the rest of the slice
    // counts ties as it compares
    // (a row of ties, such as all zeros with tau = 0, otherwise sends every
    // vector through the survivor code)
    if (more && !full) {
      while (q_cnt) drain_queue(q_cnt < 64u ? q_cnt : 64u);   // (queued in this mode)
      while (more) {
        u32x4 v[FILTER_UNROLL];
#pragma unroll
        for (uint32_t u = 0; u < FILTER_UNROLL; ++u) v[u] = nxt[u];
        const size_t vc = vi;
        vi += sstep;
        more = step_ok(vi);
        if (more) {
#pragma unroll
          for (uint32_t u = 0; u < FILTER_UNROLL; ++u)
            nxt[u] = __builtin_nontemporal_load(vp + vi + u * stride);
        }
        scan_step_dense(v, vc, !more);
        if (full) break;
      }
    }
  } else {
    for (; (vi - lane) + 63 + (FILTER_UNROLL - 1) * stride < vend; vi += FILTER_UNROLL * stride) {
      u32x4 v[FILTER_UNROLL];
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) v[u] = vp[vi + u * stride];
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) vec_survivors(v[u], vi + u * stride, true);
      if (full) break;
    }
  }
  if (full) vi = vend + lane;   // skip the remainder as well
  // Remainder of the slice: the bound differs between lanes, so iterate on
  // the wave's first lane index to keep ballots wave-uniform.
  for (;;) {
    const size_t wave_first = vi - lane;
    if (wave_first >= vend) break;
    const bool valid = vi < vend;
    const u32x4 v = valid ? vp[vi] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t e0 = head + (uint32_t)vi * D::VEC;
    bool any = false;
#pragma unroll
    for (int e = 0; e < D::VEC; ++e) {
      uint32_t raw;
      if constexpr (DT == DT_BF16) raw = (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xFFFFu);
      else raw = v[e];
      any = any || (valid && pass_of(raw));
    }
    if (ballot(any) != 0) {
#pragma unroll
      for (int e = 0; e < D::VEC; ++e) {
        uint32_t raw;
        if constexpr (DT == DT_BF16) raw = (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xFFFFu);
        else raw = v[e];
        push_one(valid && pass_of(raw), raw, e0 + e);
      }
    }
    vi += stride;
  }
  // Head and tail elements: the first wave of workgroup 0.
  if (blockIdx.x == 0 && w == 0) {
    const uint32_t nt = n - tail0;
    for (uint32_t base = 0; base < head + nt; base += 64) {
      const uint32_t j = base + lane;
      const bool ok = j < head + nt;
      uint32_t idx = 0, raw = 0;
      if (ok) {
        idx = (j < head) ? j : tail0 + (j - head);
        raw = load_raw<DT>(rowp, idx);
      }
      push_one(ok && pass_of(raw), raw, idx);
    }
  }

  if (traced && threadIdx.x == 0) wg_trace[2 * (size_t)lwg + 1] = __builtin_amdgcn_s_memrealtime();

  // Workgroup flush: one atomic per buffer, one for the tie count, and one
  // for the above-tau total (the staged entries plus those the waves
  // flushed on the way; the count the finish kernel reads, which no other
  // kernel rewrites).
  ties = wave_sum_u32(ties);
  if (lane == 0) {
    s_fill[w] = sg.fill;
    s_tfill[w] = tg.fill;
    s_ties[w] = ties;
    s_flushed[w] = sg.flushed;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t total = 0, ttotal = 0, tcount = 0, earlier = 0;
    for (uint32_t i = 0; i < FILTER_WAVES; ++i) {
      total += s_fill[i];
      ttotal += s_tfill[i];
      tcount += s_ties[i];
      earlier += s_flushed[i];
    }
    s_base = total ? atomicAdd(&st->count, total) : 0u;
    s_tbase = ttotal ? atomicAdd(&rc->tslots, ttotal) : 0u;
    if (tcount) atomicAdd(&rc->ties, tcount);
    if (total + earlier) atomicAdd(&rc->above, total + earlier);
  }
  __syncthreads();
  uint32_t off = s_base, toff = s_tbase;
  for (uint32_t i = 0; i < w; ++i) {
    off += s_fill[i];
    toff += s_tfill[i];
  }
  uint32_t km = 0;
  for (uint32_t i = lane; i < sg.fill; i += 64) {
    const uint32_t pos = off + i;
    if (pos < cap) sg.buf[pos] = sg.stage[i];
    const uint32_t key = (uint32_t)(sg.stage[i] >> B);
    km = key > km ? key : km;
  }
  for (uint32_t i = lane; i < tg.fill; i += 64) {
    const uint32_t pos = toff + i;
    if (pos < cap) tg.buf[pos] = tg.stage[i];
  }
  if (track_kmax) {   // one atomic per workgroup
    km = wave_max_u32(km);
    km = sg.km > km ? sg.km : km;
    if (lane == 0 && km) atomicMax(&s_km, km);
    __syncthreads();
    if (tid == 0 && s_km) atomicMax(&rc->kmax, s_km);
  }
}

template <int DT>
__global__ __launch_bounds__(FILTER_THREADS) void k_filter(TK_FILTER_PARAMS) {
  filter_body<DT, false>(TK_FILTER_ARGS);
}
template <int DT>
__global__ __launch_bounds__(FILTER_THREADS) void k_filter_ahead3(TK_FILTER_PARAMS) {
  filter_body<DT, true>(TK_FILTER_ARGS);
}
#undef TK_FILTER_PARAMS
#undef TK_FILTER_ARGS

// ======================================================================
// Detection (Prof-K section 3, stage 4): R < k is a recall failure, R > M an
// overflow; either sends the row to the exact path.  With the survivors split
// at tau (G strictly above, E equal):
//   G > cap          overflow
//   G >= k           accepted: the k winners lie among the G, ties unused
//   G + E > cap      the ties needed do not fit: overflow
//   G + E >= k       accepted with every tie (all E were stored, E <= cap - G)
//   G + E >= k_eff   relaxed recall (k_eff < k): fewer than k reach tau, and
//                    every one of them is a top-k element; they are kept
//   otherwise        recall failure
// ======================================================================
enum : uint32_t { V_FAIL = 0, V_OK = 1, V_OK_TIES = 2, V_PARTIAL = 3 };

__device__ __forceinline__ uint32_t sampled_verdict(uint32_t G, uint32_t E, uint32_t k,
                                                    uint32_t k_eff, uint32_t cap) {
  if (G > cap) return V_FAIL;
  if (G >= k) return V_OK;
  const uint64_t R = (uint64_t)G + E;
  if (R > cap) return V_FAIL;
  if (R >= k) return V_OK_TIES;
  if (R >= k_eff) return V_PARTIAL;
  return V_FAIL;
}

// Leaves count and ties alone: other workgroups may still be reading them to
// reach the same verdict (the exact route resets count once its threshold is
// known).
__device__ __forceinline__ void start_exact(RowState* st, uint32_t k, uint32_t path) {
  st->status = ST_EXACT;
  st->path = path;
  st->need = k;
  st->above = 0;
  st->prefix = 0;
  st->nbits = 0;
  st->passes = 0;
}

// Rows sent to the exact route are listed for the exact-route kernel.
__device__ __forceinline__ void flag_row(CallState* cs, uint32_t* flagged, uint32_t row) {
  const uint32_t slot = atomicAdd(&cs->nflag, 1u);
  atomicAdd(&cs->nactive, 1u);
  flagged[slot] = row;
}

__global__ void k_check(RowState* __restrict__ states, const RowCtr* __restrict__ rctr,
                        CallState* __restrict__ cs, uint32_t* __restrict__ flagged, uint32_t rows,
                        uint32_t k, uint32_t k_eff, uint32_t cap) {
  const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  RowState* st = states + row;
  if (st->status != ST_FILTER) return;
  const uint32_t G = rctr[row].above, E = rctr[row].ties;
  if (sampled_verdict(G, E, k, k_eff, cap) == V_FAIL) {
    st->r_sampled = G + E;
    st->ties = E;
    start_exact(st, k, PATH_FALLBACK);
    flag_row(cs, flagged, row);
  }
}

// The exact route's first kernel: the call's set-up (call record, stamp)
// and every row listed.
__global__ void k_setup_exact(RowState* __restrict__ states, CallState* __restrict__ cs,
                              uint32_t* __restrict__ flagged, uint32_t rows, uint32_t k,
                              WsHeader* hdr, uint64_t sig) {
  const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  RowState* st = states + row;
  start_exact(st, k, PATH_EXACT);
  st->r_sampled = 0;
  st->tau_key = 0;
  st->ties = 0;
  st->tau_route = TAU_NONE;
  flagged[row] = row;
  if (row == 0) {
    reset_call(cs);
    stamp_invalidate(hdr, sig);
    cs->nflag = rows;
    cs->nactive = rows;
  }
}
