// Sampler and threshold kernels (k_sample, k_tau).
// A part of topk_kernels.hip, included there in order inside namespace tk;
// it relies on the definitions of the parts before it and is not a
// stand-alone header.
#pragma once

// ======================================================================
// Sampler: S indices drawn without replacement (Prof-K, section 3, stage 1).
// The first S images of a keyed permutation of [0, n): a balanced 4-round
// Feistel network over 2h bits whose round function is the SplitMix64 output
// mixer (Steele, Lea & Flood 2014), walked back into [0, n) ("cycle walking",
// Black & Rogaway 2002).  Round keys for (seed, row) are outputs 4*row..4*row+3
// of the SplitMix64 stream seeded with `seed`.
// ======================================================================
__device__ __forceinline__ uint64_t sm64_finalize(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

struct Feistel {
  uint64_t rk[4];
  uint64_t mask;
  uint32_t h;
  __device__ Feistel(uint64_t seed, uint64_t row, uint32_t half_bits) {
    h = half_bits;
    mask = (1ull << h) - 1ull;
    const uint64_t gamma = 0x9E3779B97F4A7C15ull;
#pragma unroll
    for (int r = 0; r < 4; ++r) rk[r] = sm64_finalize(seed + (4ull * row + (uint64_t)r + 1ull) * gamma);
  }
  __device__ uint64_t apply(uint64_t x) const {
    uint64_t L = x >> h, R = x & mask;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint64_t t = L ^ (sm64_finalize(R ^ rk[r]) & mask);
      L = R;
      R = t;
    }
    return (L << h) | R;
  }
};

// Sample keys also land in an 11-bit histogram of their top bits (LDS per
// workgroup, merged into the row's global histogram), the first level of the
// threshold's radix select.
constexpr uint32_t SH_BITS = 11;
constexpr uint32_t SH_BINS = 1u << SH_BITS;

// Small threshold ranks (t <= TOPT): every sampler workgroup keeps only its
// own largest keys, sorted largest first and zero-padded (a bitonic network
// over each wave's lanes, then two bitonic merges of the wave lists): its t
// largest for t <= TOPT_EXTRACT, its TOPT largest above, and tau is selected
// from those lists instead of all S keys (by every filter workgroup in its
// prologue when there are few, else by k_tau).  Their union holds the t
// largest sampled keys, and longer lists or padding keys of 0 cannot change
// the t-th largest, so tau is unchanged.  (Letting the last sampler
// workgroup select saves the launch but needs an agent-scope release fence
// in every workgroup: measured slower, much slower with many rows.
// Extracting the t largest one at a time measured as fast up to t = 2 and
// slower above: 17.8 us instead of 7.8 on 2^28 bf16 with t = 32.)
constexpr uint32_t TOPT = 32;
constexpr uint32_t TOPT_EXTRACT = 8;   // up to here the lists hold t keys, above TOPT
constexpr uint32_t SAMPLE_THREADS = 256;
static_assert(SAMPLE_THREADS == 256 && TOPT == 32, "the sorted path merges four wave lists of 32");

// The value of lane (this lane ^ J) for J = 1, 2, ..., 32, without the LDS
// crossbar for J <= 8: DPP moves (quad permutations for 1 and 2, row shifts
// for 4, a row rotation for 8), a swizzle for 16 and a half-wave swap for 32
// (each checked against a shuffle on the GPU, all 64 lanes).  Each DPP move
// is taken into a temporary (the empty asm, not volatile, so independent
// networks still interleave) before it is combined, so that no DPP-modified
// arithmetic is formed from it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
  asm("" : "+v"(r));
  return r;
}
template <uint32_t J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (J == 1) {
    return dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  } else if constexpr (J == 2) {
    return dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  } else if constexpr (J == 4) {
    const uint32_t a = dpp_mov<0x104>(v), b = dpp_mov<0x114>(v);   // row_shl:4, row_shr:4
    return (lane_id() & 4u) ? b : a;
  } else if constexpr (J == 8) {
    return dpp_mov<0x128>(v);   // row_ror:8
  } else if constexpr (J == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);   // swap 16-lane halves
  } else {
    static_assert(J == 32, "lane strides 1 to 32");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // swap 32-lane halves
    return lane_id() < 32 ? r[1] : r[0];
  }
}

// Batcher's bitonic network over a wave's 64 lanes, one compare-exchange
// stage per template step (partner lane ^ J; runs of K alternate descending
// and ascending so that each pair of runs is bitonic for the next K; the last
// run, K = 64, descends).
template <uint32_t K, uint32_t J>
__device__ __forceinline__ uint32_t bitonic_sort_steps(uint32_t v) {
  const uint32_t l = lane_id();
  const uint32_t p = xor_lane<J>(v);
  const bool desc = (l & K) == 0u, low = (l & J) == 0u;
  const uint32_t mx = v > p ? v : p, mn = v > p ? p : v;
  v = (low == desc) ? mx : mn;
  if constexpr (J > 1) return bitonic_sort_steps<K, J / 2>(v);
  else if constexpr (K < 64) return bitonic_sort_steps<2 * K, K>(v);
  else return v;
}
template <uint32_t J>
__device__ __forceinline__ uint32_t bitonic_merge_steps(uint32_t v) {
  const uint32_t p = xor_lane<J>(v);
  const uint32_t mx = v > p ? v : p, mn = v > p ? p : v;
  v = (lane_id() & J) == 0u ? mx : mn;
  if constexpr (J > 1) return bitonic_merge_steps<J / 2>(v);
  else return v;
}

// One wave's 64 values sorted largest first (lane 0 the largest).
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v) { return bitonic_sort_steps<2, 1>(v); }

// A bitonic sequence over the wave's 64 lanes sorted largest first.
__device__ __forceinline__ uint32_t wave_merge_desc(uint32_t v) { return bitonic_merge_steps<32>(v); }

// The 32 largest of the workgroup's values (one per thread, 0 for none),
// largest first, into out[0..32).  s_l: 128 words, s_m: 64 words.  Every
// thread calls it.
__device__ __forceinline__ void block_top32_sorted(uint32_t v, uint32_t* s_l, uint32_t* s_m,
                                                   uint32_t* out) {
  const uint32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63u;
  v = wave_sort_desc(v);
  if (lane < 32) s_l[w * 32 + lane] = v;
  __syncthreads();
  if (w < 2) {   // lists 2w and 2w + 1: the second one reversed makes a bitonic sequence
    uint32_t x = lane < 32 ? s_l[2 * w * 32 + lane] : s_l[(2 * w + 1) * 32 + (63 - lane)];
    x = wave_merge_desc(x);
    if (lane < 32) s_m[w * 32 + lane] = x;
  }
  __syncthreads();
  if (w == 0) {
    uint32_t x = lane < 32 ? s_m[lane] : s_m[32 + (63 - lane)];
    x = wave_merge_desc(x);
    if (lane < 32) out[lane] = x;
  }
  __syncthreads();
}

// The t largest alive values of the wave (with multiplicity), largest first,
// written by lane 0 to out[0..); returns how many (wave-uniform).
__device__ __forceinline__ uint32_t wave_top_t(uint32_t v, bool alive, uint32_t t, uint32_t* out) {
  uint32_t c = 0;
  for (; c < t; ++c) {
    if (ballot(alive) == 0) break;
    const uint32_t m = wave_max_u32(alive ? v : 0u);
    const uint64_t hit = ballot(alive && v == m);
    if (lane_id() == (uint32_t)__builtin_ctzll(hit)) alive = false;
    if (lane_id() == 0) out[c] = m;
  }
  return c;
}

// The same with four values per lane, v[0..cnt) sorted largest first: each
// round takes the largest head and advances that lane.
__device__ __forceinline__ uint32_t wave_top_t4(const uint32_t (&v)[4], uint32_t cnt, uint32_t t,
                                                uint32_t* out) {
  uint32_t c = 0, cur = 0;
  for (; c < t; ++c) {
    const bool alive = cur < cnt;
    if (ballot(alive) == 0) break;
    const uint32_t head = cur == 0 ? v[0] : cur == 1 ? v[1] : cur == 2 ? v[2] : v[3];
    const uint32_t m = wave_max_u32(alive ? head : 0u);
    const uint64_t hit = ballot(alive && head == m);
    if (lane_id() == (uint32_t)__builtin_ctzll(hit)) ++cur;
    if (lane_id() == 0) out[c] = m;
  }
  return c;
}

// The t largest of up to four values per thread over a workgroup of NW
// waves (t <= CAP): per-wave lists, then one wave merges them.  s_wl: NW *
// CAP words, s_wc: NW + 1 words, out: CAP words; returns the length.
template <uint32_t NW, uint32_t CAP>
__device__ __forceinline__ uint32_t block_top_t4(uint32_t (&v)[4], uint32_t cnt, uint32_t t,
                                                 uint32_t* s_wl, uint32_t* s_wc, uint32_t* out) {
  static_assert(NW * CAP <= 64, "one wave merges the wave lists");
  const uint32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63u;
  auto cswap = [&](int a, int b) {
    const uint32_t hi = v[a] > v[b] ? v[a] : v[b], lo = v[a] > v[b] ? v[b] : v[a];
    v[a] = hi;
    v[b] = lo;
  };
  // largest first; the cnt valid values must be the largest (invalid = 0)
  cswap(0, 1);
  cswap(2, 3);
  cswap(0, 2);
  cswap(1, 3);
  cswap(1, 2);
  const uint32_t c = wave_top_t4(v, cnt, t, s_wl + w * CAP);
  if (lane == 0) s_wc[w] = c;
  __syncthreads();
  if (w == 0) {
    const uint32_t q = lane / CAP, i = lane % CAP;
    const bool al = q < NW && i < s_wc[q];
    const uint32_t x = al ? s_wl[q * CAP + i] : 0u;
    const uint32_t m = wave_top_t(x, al, t, out);
    if (lane == 0) s_wc[NW] = m;
  }
  __syncthreads();
  return s_wc[NW];
}

// Row setup for the sampled route (threshold known).
__device__ __forceinline__ void start_sampled_row(RowState* st, RowCtr* rc, uint32_t tau,
                                                  uint32_t route) {
  st->status = ST_FILTER;
  st->tau_route = route;
  st->tau_key = tau;
  st->count = 0;
  st->ties = 0;
  st->r_sampled = 0;
  rc->ties = 0;
  rc->tslots = 0;
  rc->kmax = 0;
  rc->above = 0;
  st->path = PATH_SAMPLED;
  st->passes = 0;
  st->kmax = 0;
}

// The first kernel of a sampled call also does the call's set-up: the call
// record to zero, and the workspace stamp cleared unless it is this layout's.
__device__ __forceinline__ void call_prologue(CallState* cs, WsHeader* hdr, uint64_t sig) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    reset_call(cs);
    stamp_invalidate(hdr, sig);
  }
}

// Writes the keys k_tau selects from: all S sample keys and their 11-bit
// histogram (lists = 0), or each workgroup's t largest at g * t, for t above
// TOPT_EXTRACT its TOPT largest at g * TOPT, sorted (lists = 1;
// k_tau histograms those itself: the largest keys of every workgroup share
// a few top bins, and global atomics on them would serialise).  The global
// histogram is used only when the workspace stamp says it starts at zero;
// otherwise k_tau histograms the keys itself.
template <int DT>
__global__ __launch_bounds__(SAMPLE_THREADS) void k_sample(
    const void* __restrict__ values, uint64_t seed, uint32_t* __restrict__ skeys, uint32_t n,
    uint32_t S, uint32_t SP, uint32_t half_bits, uint32_t lists, uint32_t t, uint32_t route,
    RowState* __restrict__ states, RowCtr* __restrict__ rctr, CallState* cs, WsHeader* hdr,
    uint32_t* __restrict__ shist, uint64_t sig) {
  // (the arguments the gather needs come first: the first 14 words of the
  // argument block arrive in scalar registers with the launch)
  __shared__ uint32_t h[SH_BINS];
  __shared__ uint32_t s_wl[4 * TOPT], s_out[TOPT], s_m[2 * TOPT];
  const uint32_t row = blockIdx.y, tid = threadIdx.x;
  const uint32_t j = blockIdx.x * SAMPLE_THREADS + tid;
  const bool in = j < S;
  // The gather goes out first, unconditionally (a lane past S reads element
  // 0 and drops it): the rest of the set-up overlaps its latency, and the
  // empty asm keeps the compiler from moving that set-up's stores, and the
  // waits for their addresses, in front of it.
  uint64_t x = 0;
  if (in) {
    const Feistel f(seed, row, half_bits);
    x = f.apply(j);
    while (x >= n) x = f.apply(x);   // ends: the cycle through j < n returns below n
  }
  const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
  const uint32_t raw = load_raw<DT>(rowp, (uint32_t)x);
  asm volatile("" ::: "memory");
  const bool gh_ok = !lists && hdr->stamp == sig;   // read before the prologue may clear it
  call_prologue(cs, hdr, sig);
  // the filter selects tau itself: start the row here (tau set there)
  if (states && blockIdx.x == 0 && tid == 0)
    start_sampled_row(states + row, rctr + row, 0u, route);
  uint32_t* gh = shist + (size_t)row * SH_BINS;
  if (gh_ok) {
    for (uint32_t i = tid; i < SH_BINS; i += SAMPLE_THREADS) h[i] = 0;
    __syncthreads();
  }
  uint32_t key = 0;
  if (in) {
    key = Dt<DT>::key(raw);
    if (!lists) {
      skeys[(size_t)row * SP + j] = key;
      if (gh_ok) atomicAdd(&h[key >> (Dt<DT>::KB - SH_BITS)], 1u);
    }
  }
  if (!lists) {
    if (!gh_ok) return;
    __syncthreads();
    for (uint32_t i = tid; i < SH_BINS; i += SAMPLE_THREADS)
      if (h[i]) atomicAdd(&gh[i], h[i]);
    return;
  }
  // this workgroup's t largest keys, zero-padded
  // (sorted by Batcher's network even for t <= TOPT_EXTRACT: as fast as
  // extracting t keys one at a time up to t = 2, faster above; t > TOPT_EXTRACT
  // keeps all TOPT sorted keys: the union of these longer lists still holds
  // the t largest sampled keys, each list its own largest first)
  block_top32_sorted(j < S ? key : 0u, s_wl, s_m, s_out);
  const uint32_t len = t <= TOPT_EXTRACT ? t : TOPT;
  if (tid < len) skeys[(size_t)row * SP + blockIdx.x * len + tid] = s_out[tid];
}

// ======================================================================
// Threshold (Prof-K section 3, stage 2): tau = the t-th largest sampled key,
// found by a workgroup radix select instead of a sort.  Also starts the row.
// ======================================================================
struct KeySrc {
  const uint32_t* p;
  __device__ uint64_t operator()(uint32_t i) const { return p[i]; }
};

constexpr uint32_t SEL_THREADS = 1024;
constexpr uint32_t CAND_CAP = 8192;   // LDS candidates (64 KB)

// One workgroup per row.  The sample keys are loaded into registers first
// (TAU_VEC 16-byte words per thread), so their loads overlap the histogram:
// the row's global one (built by the sampler), or for few keys one built
// here.  One wave finds the bin holding rank t; the keys of that bin go
// from registers to LDS (one slot reservation per wave), and the select
// finishes there.  Longer key lists take a streaming pass instead.
// Sample-key rows are padded to a multiple of 4 keys (SP = padded length).
constexpr uint32_t TAU_VEC = 8;
__global__ __launch_bounds__(SEL_THREADS) void k_tau(const uint32_t* __restrict__ skeys, uint32_t S,
                                                     uint32_t SP, uint32_t t, uint32_t KB,
                                                     uint32_t* __restrict__ shist,
                                                     uint32_t lists,
                                                     RowState* __restrict__ states,
                                                     RowCtr* __restrict__ rctr,
                                                     const WsHeader* hdr, uint64_t sig) {
  static_assert(SH_BINS == 2048, "one wave searches 2048 bins");
  __shared__ __align__(16) uint32_t s_hist[SH_BINS];
  __shared__ uint32_t s_misc[8];
  __shared__ uint32_t s_tmp[16];
  __shared__ uint64_t s_cand[CAND_CAP];
  const uint32_t row = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const uint32_t sh = KB - SH_BITS;
  const uint32_t* keys = skeys + (size_t)row * SP;
  const u32x4* kv4 = reinterpret_cast<const u32x4*>(keys);
  const uint32_t nv = (S + 3) / 4;
  const bool regs = nv <= TAU_VEC * nt;   // every key fits the registers
  // the sampler's global histogram, unless it was not usable (stamp)
  const bool own_hist = lists || hdr->stamp != sig;
  uint32_t route = lists ? TAU_KTAU_LISTS : (regs ? TAU_KTAU_REGS : TAU_KTAU_STREAM);
  u32x4 kv[TAU_VEC];
#pragma unroll
  for (uint32_t j = 0; j < TAU_VEC; ++j) {
    const uint32_t v = j * nt + tid;
    kv[j] = (regs && v < nv) ? kv4[v] : u32x4{0u, 0u, 0u, 0u};
  }
  auto valid = [&](uint32_t j, int q) { return (j * nt + tid) * 4u + (uint32_t)q < S; };
  if (tid == 0) s_misc[3] = 0;
  if (own_hist) {   // few keys, or no usable global histogram: histogram them here
    for (uint32_t i = tid; i < SH_BINS; i += nt) s_hist[i] = 0;
    if (!lists) {   // leave the global histogram zero for the stamp
      uint32_t* gh = shist + (size_t)row * SH_BINS;
      for (uint32_t i = tid; i < SH_BINS; i += nt) gh[i] = 0;
    }
    __syncthreads();
    if (regs) {
#pragma unroll
      for (uint32_t j = 0; j < TAU_VEC; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) hist_add(s_hist, kv[j][q] >> sh, valid(j, q));
    } else {
      for (uint32_t i = tid; i < S; i += nt) atomicAdd(&s_hist[keys[i] >> sh], 1u);
    }
  } else {
    uint32_t* gh = shist + (size_t)row * SH_BINS;
    for (uint32_t i = tid; i < SH_BINS; i += nt) {
      s_hist[i] = gh[i];
      gh[i] = 0;                      // ready for the next call
    }
  }
  __syncthreads();
  if (tid < 64) wave_find_bucket_2048(s_hist, t, s_misc);
  __syncthreads();
  const uint32_t b = s_misc[0], acc = s_misc[1], hb = s_misc[2];
  KeySrc src{keys};
  SelectStart st0;
  st0.prefix = (uint64_t)b << sh;
  st0.nb = SH_BITS;
  st0.need = t - acc;
  st0.above = acc;
  if (hb <= CAND_CAP) {
    // the boundary bin's keys into LDS
    if (regs) {
      uint32_t mine = 0;
#pragma unroll
      for (uint32_t j = 0; j < TAU_VEC; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) mine += (valid(j, q) && (kv[j][q] >> sh) == b) ? 1u : 0u;
      const uint32_t incl = wave_incl_sum(mine);
      const uint32_t wtot = wave_bcast(incl, 63u);
      uint32_t wbase = 0;
      if ((tid & 63u) == 0 && wtot) wbase = atomicAdd(&s_misc[3], wtot);
      uint32_t pos = wave_bcast(wbase, 0u) + incl - mine;
#pragma unroll
      for (uint32_t j = 0; j < TAU_VEC; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (valid(j, q) && (kv[j][q] >> sh) == b) {
            if (pos < CAND_CAP) s_cand[pos] = kv[j][q];
            ++pos;
          }
    } else {
      for_batched_i<12, u32x4>(
          nv, [&](uint32_t i) { return kv4[i]; },
          [&](const u32x4& v, bool ok, uint32_t i) {
            bool in[4];
            bool any = false;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              in[q] = ok && (i * 4 + q) < S && (v[q] >> sh) == b;
              any = any || in[q];
            }
            if (ballot(any) == 0) return;   // the usual case: no key of the bin
#pragma unroll
            for (int q = 0; q < 4; ++q) lds_append(s_cand, &s_misc[3], CAND_CAP, v[q], in[q]);
          });
    }
    __syncthreads();
    st0.m = s_misc[3] < CAND_CAP ? s_misc[3] : CAND_CAP;
    st0.in_lds = true;
  }
  uint32_t tau;
  if (!st0.in_lds) route |= TAU_BIN_STREAMED;
  else if (st0.m > nt / 4) route |= TAU_BIN_RADIX;
  if (st0.in_lds && st0.m <= nt / 4) {
    // a small bin: the wanted key is the one whose rank inside it (larger
    // keys, then equal keys earlier in the list) is need - 1; four lanes
    // share each key, each counting a quarter of the list
    const uint32_t i = tid >> 2, q = tid & 3u;
    const uint64_t mine = i < st0.m ? s_cand[i] : 0ull;
    uint32_t r = 0;
    for (uint32_t j = q; j < st0.m; j += 4) {
      const uint64_t o = s_cand[j];
      r += (o > mine || (o == mine && j < i)) ? 1u : 0u;
    }
    r += dpp_take<0xB1, 0xf>(r);
    r += dpp_take<0x4E, 0xf>(r);
    if (q == 0 && i < st0.m && r == st0.need - 1) s_misc[5] = (uint32_t)mine;
    __syncthreads();
    tau = s_misc[5];
  } else {
    __syncthreads();   // every thread has read the bin
    tau = (uint32_t)block_select_from(src, S, KB, st0, 0u, s_hist, s_misc, s_cand, CAND_CAP).thr;
  }
  if (tid == 0) start_sampled_row(states + row, rctr + row, tau, route);
}

// The caller's threshold for every row (topk_params.use_force_tau): the
// call's set-up and the row starts that the sampler and k_tau would do.
__global__ __launch_bounds__(SAMPLE_THREADS) void k_force_tau(RowState* __restrict__ states,
                                                              RowCtr* __restrict__ rctr,
                                                              CallState* cs, WsHeader* hdr,
                                                              uint64_t sig, uint32_t tau) {
  call_prologue(cs, hdr, sig);
  if (blockIdx.x == 0 && threadIdx.x == 0)
    start_sampled_row(states + blockIdx.y, rctr + blockIdx.y, tau, TAU_FORCED);
}
