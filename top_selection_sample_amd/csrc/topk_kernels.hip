// HIP kernels of the exact top-k engine for gfx950 (MI355X), and their
// launchers.  The pipeline follows the four stages of the Prof-K paper
// (section 3, "The Prof-K Algorithm"): sampling, threshold estimation,
// filtering into a bounded candidate buffer, exact refinement; with the
// fallback to an exact selection over the full row when fewer than k
// candidates survive or the buffer overflows.
//
// Kernels (one row = one independent selection; grids are (tiles, rows)):
//   k_sample       S sample keys per row through a keyed permutation
//   k_tau          workgroup radix select of the t-th largest sample key
//   k_filter       the streaming pass: keep composites with key >= tau
//   k_check        many rows: list the rows whose candidate count fails
//   k_setup_exact  rows that start on the exact path
//   k_finish       the check, the refine of every accepted row (small k: select,
//                  sort and write the k winners), and the exact route for the
//                  failed rows, in one persistent launch
//   k_exact_small  small rows: the whole exact selection in one workgroup
//   k_tile_sort / k_merge / k_output   large k: sort all candidates
#include "topk_device.hpp"
#include "topk_launch.hpp"
#include "topk_select.hpp"

namespace tk {

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
// own t largest keys (zero-padded to t), and k_tau selects from those G * t
// keys instead of all S.  Their union holds the t largest sampled keys, and
// padding keys of 0 cannot raise the t-th largest, so tau is unchanged.
// (Letting the last sampler workgroup select saves the launch but needs an
// agent-scope release fence in every workgroup: measured slower, much
// slower with many rows.)
constexpr uint32_t TOPT = 16;
constexpr uint32_t SAMPLE_THREADS = 256;
static_assert((SAMPLE_THREADS / 64) * TOPT <= 64, "one wave merges the wave lists");

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

// The same over the whole workgroup (SAMPLE_THREADS); the result in out
// (TOPT words), its length returned.  s_wl: 4 * TOPT words, s_wc: 5 words.
__device__ __forceinline__ uint32_t block_top_t(uint32_t v, bool alive, uint32_t t, uint32_t* s_wl,
                                                uint32_t* s_wc, uint32_t* out) {
  const uint32_t tid = threadIdx.x, w = tid >> 6, lane = tid & 63u;
  const uint32_t c = wave_top_t(v, alive, t, s_wl + w * TOPT);
  if (lane == 0) s_wc[w] = c;
  __syncthreads();
  if (w == 0) {
    const uint32_t q = lane / TOPT, i = lane % TOPT;
    const bool al = q < SAMPLE_THREADS / 64 && i < s_wc[q];
    const uint32_t x = al ? s_wl[q * TOPT + i] : 0u;
    const uint32_t cnt = wave_top_t(x, al, t, out);
    if (lane == 0) s_wc[4] = cnt;
  }
  __syncthreads();
  return s_wc[4];
}

// Row setup for the sampled route (threshold known).
__device__ __forceinline__ void start_sampled_row(RowState* st, RowCtr* rc, uint32_t tau) {
  st->status = ST_FILTER;
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

// Writes the keys k_tau selects from: all S sample keys and their 11-bit
// histogram (lists = 0), or each workgroup's t largest at g * t (lists = 1;
// k_tau histograms those itself: the largest keys of every workgroup share
// a few top bins, and global atomics on them would serialise).
template <int DT>
__global__ __launch_bounds__(SAMPLE_THREADS) void k_sample(
    const void* __restrict__ values, uint32_t n, uint32_t S, uint32_t SP, uint64_t seed,
    uint32_t half_bits, uint32_t* __restrict__ skeys, uint32_t* __restrict__ shist, uint32_t lists,
    uint32_t t, RowState* __restrict__ states, RowCtr* __restrict__ rctr) {
  __shared__ uint32_t h[SH_BINS];
  __shared__ uint32_t s_wl[4 * TOPT], s_wc[8], s_out[TOPT];
  const uint32_t row = blockIdx.y, tid = threadIdx.x;
  // the filter selects tau itself: start the row here (tau set there)
  if (states && blockIdx.x == 0 && tid == 0) start_sampled_row(states + row, rctr + row, 0u);
  uint32_t* gh = shist + (size_t)row * SH_BINS;
  if (!lists) {
    for (uint32_t i = tid; i < SH_BINS; i += SAMPLE_THREADS) h[i] = 0;
    __syncthreads();
  }
  const uint32_t j = blockIdx.x * SAMPLE_THREADS + tid;
  uint32_t key = 0;
  if (j < S) {
    const Feistel f(seed, row, half_bits);
    uint64_t x = f.apply(j);
    while (x >= n) x = f.apply(x);   // ends: the cycle through j < n returns below n
    const char* rowp = static_cast<const char*>(values) + (size_t)row * n * Dt<DT>::ES;
    key = Dt<DT>::key(load_raw<DT>(rowp, (uint32_t)x));
    if (!lists) {
      skeys[(size_t)row * SP + j] = key;
      atomicAdd(&h[key >> (Dt<DT>::KB - SH_BITS)], 1u);
    }
  }
  if (!lists) {
    __syncthreads();
    for (uint32_t i = tid; i < SH_BINS; i += SAMPLE_THREADS)
      if (h[i]) atomicAdd(&gh[i], h[i]);
    return;
  }
  // this workgroup's t largest keys, zero-padded
  const uint32_t c = block_top_t(key, j < S, t, s_wl, s_wc, s_out);
  if (tid < t) skeys[(size_t)row * SP + blockIdx.x * t + tid] = tid < c ? s_out[tid] : 0u;
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
                                                     uint32_t own_hist,
                                                     RowState* __restrict__ states,
                                                     RowCtr* __restrict__ rctr) {
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
  u32x4 kv[TAU_VEC];
#pragma unroll
  for (uint32_t j = 0; j < TAU_VEC; ++j) {
    const uint32_t v = j * nt + tid;
    kv[j] = (regs && v < nv) ? kv4[v] : u32x4{0u, 0u, 0u, 0u};
  }
  auto valid = [&](uint32_t j, int q) { return (j * nt + tid) * 4u + (uint32_t)q < S; };
  if (tid == 0) s_misc[3] = 0;
  if (own_hist) {   // few keys: histogram them here
    for (uint32_t i = tid; i < SH_BINS; i += nt) s_hist[i] = 0;
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
  if (tid == 0) start_sampled_row(states + row, rctr + row, tau);
}

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
constexpr uint32_t STAGE_SLOTS = 256;
constexpr uint32_t FILTER_UNROLL = 4;

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

template <int DT>
__global__ __launch_bounds__(FILTER_THREADS) void k_filter(
    const void* __restrict__ values, uint32_t n, RowState* __restrict__ states,
    RowCtr* __restrict__ rctr, uint64_t* __restrict__ cbuf, uint64_t* __restrict__ tbuf,
    uint32_t cap, uint32_t B, uint32_t track_kmax, const uint32_t* __restrict__ tlist,
    uint32_t tlist_n, uint32_t tlist_stride, uint32_t t) {
  using D = Dt<DT>;
  const uint32_t row = blockIdx.y;
  RowState* st = states + row;
  if (st->status != ST_FILTER) return;
  Thr thr;   // set below, once tau is known

  __shared__ uint64_t s_stage[FILTER_WAVES][STAGE_SLOTS];
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
  auto vec_survivors = [&](const u32x4& v0, size_t vi_lane) {
    const u32x4 v[1] = {v0};
    auto idx_of = [&](uint32_t b) { return head + (uint32_t)vi_lane * D::VEC + b; };
    uint32_t ge = 0;
#pragma unroll
    for (uint32_t b = 0; b < D::VEC; ++b) ge |= (uint32_t)pass_of(elemvc<DT, 1>(v, b)) << b;
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

  // This workgroup's slice of the row's vectors: [vi0, vend), in steps of
  // FILTER_THREADS * FILTER_UNROLL vectors.
  const uint32_t bpr = gridDim.x;
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
  // of loads in flight.  The first step's loads go out before tau is known.
  auto step_ok = [&](size_t at) { return (at - lane) + 63 + (FILTER_UNROLL - 1) * stride < vend; };
  u32x4 nxt[FILTER_UNROLL];
  bool more = step_ok(vi);
  if (more) {
#pragma unroll
    for (uint32_t u = 0; u < FILTER_UNROLL; ++u)
      nxt[u] = __builtin_nontemporal_load(vp + vi + u * stride);
  }
  // tau: given by k_tau, or (tlist_n > 0) the t-th largest of the sampler's
  // per-workgroup top-t lists, selected here by every workgroup
  uint32_t tau;
  if (tlist_n) {
    __shared__ uint32_t s_tl[FILTER_WAVES * 8], s_tc[FILTER_WAVES + 1], s_to[8];
    const uint32_t* kl = tlist + (size_t)row * tlist_stride;
    uint32_t v[4], cnt = 0;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
      const uint32_t i = q * FILTER_THREADS + tid;
      v[q] = i < tlist_n ? kl[i] : 0u;
      cnt += i < tlist_n ? 1u : 0u;
    }
    block_top_t4<FILTER_WAVES, 8>(v, cnt, t, s_tl, s_tc, s_to);
    tau = s_to[t - 1];   // the lists hold at least t keys
    if (blockIdx.x == 0 && tid == 0) st->tau_key = tau;
  } else {
    tau = st->tau_key;
  }
  thr = make_thr<DT>(tau, 0xFFFFFFFFu);
  if (thr.kind == 0) {
    while (more) {
      u32x4 v[FILTER_UNROLL];
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) v[u] = nxt[u];
      const size_t vc = vi;
      vi += FILTER_UNROLL * stride;
      more = step_ok(vi);
      if (more) {
#pragma unroll
        for (uint32_t u = 0; u < FILTER_UNROLL; ++u)
          nxt[u] = __builtin_nontemporal_load(vp + vi + u * stride);
      }
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) {
        uint32_t any = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (DT == DT_BF16) {
            any |= (uint32_t)native_pass<DT>(v[u][q] & 0xFFFFu, thr);
            any |= (uint32_t)native_pass<DT>(v[u][q] >> 16, thr);
          } else {
            any |= (uint32_t)native_pass<DT>(v[u][q], thr);
          }
        }
        if (ballot(any != 0u) != 0) vec_survivors(v[u], vc + u * stride);
      }
      if (full) break;
    }
  } else {
    for (; (vi - lane) + 63 + (FILTER_UNROLL - 1) * stride < vend; vi += FILTER_UNROLL * stride) {
      u32x4 v[FILTER_UNROLL];
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) v[u] = vp[vi + u * stride];
#pragma unroll
      for (uint32_t u = 0; u < FILTER_UNROLL; ++u) vec_survivors(v[u], vi + u * stride);
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
  const uint32_t G = st->count, E = rctr[row].ties;
  if (sampled_verdict(G, E, k, k_eff, cap) == V_FAIL) {
    st->r_sampled = G + E;
    st->ties = E;
    start_exact(st, k, PATH_FALLBACK);
    flag_row(cs, flagged, row);
  }
}

__global__ void k_setup_exact(RowState* __restrict__ states, CallState* __restrict__ cs,
                              uint32_t* __restrict__ flagged, uint32_t rows, uint32_t k) {
  const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  RowState* st = states + row;
  start_exact(st, k, PATH_EXACT);
  st->r_sampled = 0;
  st->tau_key = 0;
  st->ties = 0;
  flagged[row] = row;
  if (row == 0) {
    cs->nflag = rows;
    cs->nactive = rows;
  }
}

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
template <int DT>
__device__ void refine_sampled(const void* __restrict__ values, uint32_t n, RowState* st,
                               const uint64_t* __restrict__ cb, uint32_t R, uint32_t lo,
                               uint32_t kmax, uint32_t k, uint32_t ks, uint32_t B, uint32_t W,
                               void* __restrict__ out_values, int64_t* __restrict__ out_idx,
                               uint32_t row, uint32_t* s_hist, uint32_t* s_misc, uint32_t* s_tmp,
                               uint64_t* s_cand, uint64_t* s_scratch) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
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
  if (tid < 64) wave_find_bucket_2048(s_hist, k, s_misc);
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
    uint32_t small_k, void* __restrict__ out_values, int64_t* __restrict__ out_idx) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_misc[8];
  __shared__ __align__(16) uint64_t s_cand[CAND_CAP];
  static_assert(CAND_CAP * 2 >= RF_RANK_MAX * 2 + RF_BINS, "bins beside the ranked candidates");
  const uint32_t row = blockIdx.x;
  RowState* st = states + row;
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
  }
}

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
// grid is one workgroup per compute unit, so all workgroups are resident
// together; every barrier wait is bounded, and a wait that gives up sets
// CallState::error instead of hanging.  The same launch first refines the
// rows whose sampled candidates passed the check, so when no row failed the
// exact route costs nothing beyond that launch.
// ======================================================================
constexpr uint32_t SPIN_LIMIT = 1u << 22;

// Arrival: a release fence (this workgroup's writes reach memory), then one
// relaxed increment of the arrival count; the last arrival acquires the
// others' writes, resets the count and bumps the generation.  Waiting polls
// the generation with relaxed loads and acquires once it has moved: an
// acquiring load per poll would invalidate the L2 at every iteration, which
// measured about four times slower on MI355X (~22 us against ~6 us per
// barrier over 256 workgroups).
__device__ void grid_barrier(CallState* cs, uint32_t G) {
  __syncthreads();
  if (threadIdx.x == 0) {
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
        __builtin_amdgcn_s_sleep(2);
        if (++spins > SPIN_LIMIT) {
          __hip_atomic_fetch_or(&cs->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  }
  __syncthreads();
}

constexpr uint32_t EX_THREADS = 1024;
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
// are the bucket:
//   k_lk_hist     bucket histogram (one LDS histogram per 4096 candidates)
//   k_lk_scatter  bucket starts (descending order), then every candidate of
//                 a bucket that starts below k goes to its bucket in aux
//   k_lk_sort     one workgroup per LK_WIN output positions sorts the buckets
//                 starting there in LDS and writes the winners directly; a
//                 bucket too large for LDS is split further in the
//                 workgroup (11-bit digits below the common prefix of its
//                 smallest and largest value, through global scratch).
// Workspace lk (u32): [rows][4096] histogram, [rows][4096] fill counters
// (both zero between calls), [rows][LK_STRIDE] bucket starts by rank
// (rank r = 4095 - bucket, so starts ascend with r; entry 4096 = the total),
// [rows][2][LK_MAXWIN] per sort window the first and last rank of the
// non-empty buckets starting in it (first = ~0: none).
// ======================================================================
constexpr uint32_t LK_BITS = 12;
constexpr uint32_t LK_BINS = 1u << LK_BITS;
constexpr uint32_t LK_STRIDE = LK_BINS + 4;
constexpr uint32_t LK_THREADS = 1024;
constexpr uint32_t LK_CHUNK = 4 * LK_THREADS;   // candidates per histogram / scatter workgroup
constexpr uint32_t LK_WIN = 1024;               // output positions per sort workgroup
constexpr uint32_t LK_LCAP = 2048;              // largest range sorted in LDS
constexpr uint32_t LK_STACK = 1024;             // pending oversized ranges per workgroup
constexpr uint32_t LK_MAXWIN = (uint32_t)(LK_CAP_MAX / LK_WIN);
static_assert(LK_WORDS_PER_ROW == 2 * LK_BINS + LK_STRIDE + 2 * LK_MAXWIN, "workspace layout");
static_assert((int64_t)LK_STACK * LK_LCAP >= LK_CAP_MAX,
              "oversized ranges are disjoint and larger than LK_LCAP, so at most "
              "LK_CAP_MAX / LK_LCAP of them are ever pending");
static_assert(LK_LCAP >= 2 * LK_WIN, "a window's small buckets fit one LDS sort");

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

// One LK_CHUNK of a row's candidates into the row's bucket histogram (lk):
// an LDS histogram, then one global atomic per non-empty bucket.  Candidate
// i is cb[i] below G and tb[i - G] from G on (the tie region, for a row
// whose ties join its candidates before they are copied over).  Every
// thread of the workgroup calls it; h: LK_BINS words of LDS.
__device__ void lk_hist_chunk(const uint64_t* __restrict__ cb, const uint64_t* __restrict__ tb,
                              uint32_t G, uint32_t R, uint32_t base, const LkDigit& g,
                              uint32_t* __restrict__ gh, uint32_t* h) {
  const uint32_t tid = threadIdx.x, nt = blockDim.x;
  for (uint32_t i = tid; i < LK_BINS; i += nt) h[i] = 0;
  uint64_t c[4];
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) {
    const uint32_t i = base + j * nt + tid;
    c[j] = i < R ? (i < G ? cb[i] : tb[i - G]) : 0ull;
  }
  __syncthreads();
#pragma unroll
  for (uint32_t j = 0; j < 4; ++j) hist_add(h, g(c[j]), base + j * nt + tid < R);
  __syncthreads();
  for (uint32_t i = tid; i < LK_BINS; i += nt)
    if (h[i]) atomicAdd(&gh[i], h[i]);
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
// k_finish builds the large-k bucket histograms of the accepted sampled rows
// and/or of the exact route's rows (the first step of the bucket sort).
enum : uint32_t { LK_HIST_SAMPLED = 1, LK_HIST_EXACT = 2 };
constexpr uint32_t FIN_SCAN_ROWS = 1024;

template <int DT>
__global__ __launch_bounds__(EX_THREADS) void k_finish(
    const void* __restrict__ values, uint32_t n, uint32_t rows, RowState* __restrict__ states,
    const RowCtr* __restrict__ rctr, CallState* __restrict__ cs, uint32_t* __restrict__ flagged,
    uint32_t* __restrict__ ghist,
    uint64_t* __restrict__ cbuf, const uint64_t* __restrict__ tbuf, uint32_t cap, uint32_t k,
    uint32_t k_eff, uint32_t B, uint32_t W, uint32_t small_k, uint32_t mode,
    void* __restrict__ out_values, int64_t* __restrict__ out_idx, uint32_t* __restrict__ lk,
    uint32_t bl, uint32_t lk_flags) {
  using D = Dt<DT>;
  __shared__ __align__(16) uint32_t s_hist[RF_BINS];
  __shared__ uint32_t s_misc[8];
  __shared__ uint32_t s_tmp[16];
  __shared__ uint64_t s_cand[RF_SORT_CAP];
  __shared__ uint32_t s_keys[RF_KCAP];
  __shared__ uint32_t s_idx[RF_SORT_CAP];
  const uint32_t G = gridDim.x, tid = threadIdx.x, w = tid >> 6;

  // FIN_SCAN (a sampled call): this workgroup's first row's state is read
  // here, in the same round trip as the check's reads below.
  const uint32_t r_first = blockIdx.x;
  const bool pre = mode == FIN_SCAN && r_first < rows;
  uint32_t f_status = 0, f_count = 0, f_ties = 0, f_kmax = 0, f_tau = 0;
  if (pre) {
    f_status = states[r_first].status;
    f_count = states[r_first].count;
    f_tau = states[r_first].tau_key;
    f_ties = rctr[r_first].ties;
    f_kmax = rctr[r_first].kmax;
  }
  static_assert(FIN_SCAN_ROWS % 32 == 0, "whole words of row bits");

  // ---- which rows failed the check (Prof-K section 3, stage 4)
  __shared__ uint32_t s_bad[FIN_SCAN_ROWS / 32];   // FIN_SCAN: one bit per row
  uint32_t nf;
  if (mode == FIN_SCAN) {
    const uint32_t words = (rows + 31) / 32;
    for (uint32_t i = tid; i < words; i += blockDim.x) s_bad[i] = 0u;
    __syncthreads();
    for (uint32_t r = tid; r < rows; r += blockDim.x) {
      const uint32_t G = __hip_atomic_load(&states[r].count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t E = rctr[r].ties;   // final: only the filter adds to it
      if (sampled_verdict(G, E, k, k_eff, cap) == V_FAIL) atomicOr(&s_bad[r >> 5], 1u << (r & 31));
    }
    __syncthreads();
    nf = 0;
    for (uint32_t i = 0; i < words; ++i) nf += __builtin_popcount(s_bad[i]);
  } else {
    nf = __hip_atomic_load(&cs->nflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        st->r_sampled = st->count + st->ties;
        start_exact(st, k, PATH_FALLBACK);
        flagged[slot] = r;
      }
      continue;
    }
    const bool fr = pre && r == r_first;
    if ((fr ? f_status : st->status) != ST_FILTER) continue;
    // an accepted row; when it needs the ties, they join its candidates
    const uint32_t G = fr ? f_count : st->count, E = fr ? f_ties : rctr[r].ties;
    const uint32_t kmx = fr ? f_kmax : rctr[r].kmax, tau = fr ? f_tau : st->tau_key;
    const uint32_t verdict = sampled_verdict(G, E, k, k_eff, cap);
    const bool ties_in = verdict == V_OK_TIES || verdict == V_PARTIAL;
    if (!fr) __syncthreads();   // every thread has read the counts
    if (ties_in) {
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
    if (ties_in) __syncthreads();   // the copied ties are visible to every thread
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
  // Large k: the bucket histograms of the accepted sampled rows (the first
  // step of the bucket sort), LK_CHUNK candidates per workgroup and step.
  // Every count read here is final: the filter's above-tau count and tie
  // count, tau and the largest key (the row's owner rewrites only the
  // RowState count, and copies the ties later; they are read from the tie
  // region).
  if (lk_flags & LK_HIST_SAMPLED) {
    const uint32_t maxch = (cap + LK_CHUNK - 1) / LK_CHUNK;
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
      lk_hist_chunk(cbuf + (size_t)r * cap, tbuf + (size_t)r * cap, Ga, R, c * LK_CHUNK, g,
                    lk + (size_t)r * LK_BINS, s_keys);
    }
  }
  if (nf == 0) return;                        // the common case: nothing more to do
  if (mode == FIN_SCAN) {
    if (blockIdx.x == 0 && tid == 0) {
      cs->nflag = nf;
      cs->nactive = nf;
    }
    grid_barrier(cs, G);   // the listed rows' states are visible to all
  }
  uint32_t ipr = (n / D::VEC + EX_ITEM_VEC - 1) / EX_ITEM_VEC;   // items per row
  if (ipr == 0) ipr = 1;
  const uint64_t total = (uint64_t)nf * ipr;
  auto sync_all = [&]() { grid_barrier(cs, G); };

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
  for (uint32_t pass = 0; pass < W / 8; ++pass) {
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
        const uint32_t row = flagged[f];
        const RowState* st = states + row;
        live = st->status == ST_EXACT;
        nb = st->nbits;
        prefix = st->prefix;
        g = row_geom<DT>(values, n, row);
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
    sync_all();
    // resolve: one workgroup per listed row
    for (uint32_t f = blockIdx.x; f < nf; f += G) {
      const uint32_t row = flagged[f];
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
    sync_all();
  }

  // ---- exact filter: every element >= the exact threshold into the buffer
  {
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
        const uint32_t row = flagged[f];
        RowState* st = states + row;
        live = st->status == ST_EXACT_READY;
        if (live) {
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
  }
  sync_all();

  // ---- refine (small k) or hand over to the sort (large k)
  for (uint32_t f = blockIdx.x; f < nf; f += G) {
    const uint32_t row = flagged[f];
    if (small_k) {
      refine_row<DT>(values, n, states, cs, flagged, cbuf, cap, k, B, W, ST_EXACT_READY,
                     out_values, out_idx, row, s_hist, s_misc, s_tmp, s_cand, s_keys, s_idx);
    } else if (tid == 0) {
      states[row].status = ST_SORT;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    // every workgroup read nflag before the first grid barrier
    cs->nflag = 0;
    cs->nactive = 0;
  }
  // Large k: the exact route's rows into their bucket histograms (their
  // count, threshold and largest key were final at the last grid barrier)
  if (!small_k && (lk_flags & LK_HIST_EXACT)) {
    const uint32_t maxch = (cap + LK_CHUNK - 1) / LK_CHUNK;
    const uint64_t npairs = (uint64_t)nf * maxch;
    for (uint64_t q = blockIdx.x; q < npairs; q += G) {
      const uint32_t row = flagged[q / maxch], c = (uint32_t)(q % maxch);
      const RowState st = states[row];
      const uint32_t R = st.count < cap ? st.count : cap;
      if ((uint64_t)c * LK_CHUNK >= R) continue;
      lk_hist_chunk(cbuf + (size_t)row * cap, cbuf + (size_t)row * cap, R, R, c * LK_CHUNK,
                    lk_digit_of(st, B, bl), lk + (size_t)row * LK_BINS, s_keys);
    }
  }
}

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
  if (blockIdx.x == 0) {   // histogram and fill counters: clean for the next call
    uint32_t* gh = lk + (size_t)row * LK_BINS;
    uint32_t* gf = lk + (size_t)(rows + row) * LK_BINS;
    for (uint32_t i = tid; i < LK_BINS; i += nt) {
      gh[i] = 0;
      gf[i] = 0;
    }
  }
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

// Measurement aid: one read of a buffer with the filter's access pattern
// (a contiguous slice per 512-thread workgroup, one workgroup per compute
// unit, FILTER_UNROLL 16-byte nontemporal loads per lane, the next step's
// loads issued before the current ones are used).  It keeps nothing but an
// XOR of the data, so its duration is the achievable time of that read
// pattern on the device, the ceiling the filter is measured against.
__global__ __launch_bounds__(FILTER_THREADS) void k_stream_read(const u32x4* __restrict__ p,
                                                                size_t nvec,
                                                                uint32_t* __restrict__ sink) {
  constexpr size_t step = (size_t)FILTER_THREADS * FILTER_UNROLL;
  const size_t per = ((nvec + gridDim.x - 1) / gridDim.x + step - 1) / step * step;
  const size_t v0 = (size_t)blockIdx.x * per;
  const size_t v1 = v0 + per < nvec ? v0 + per : nvec;
  const uint32_t tid = threadIdx.x;
  uint32_t acc = 0;
  size_t b = v0;   // the current whole step starts here
  u32x4 ra[FILTER_UNROLL], rb[FILTER_UNROLL];
  auto load = [&](u32x4 (&r)[FILTER_UNROLL], size_t at) {
#pragma unroll
    for (uint32_t u = 0; u < FILTER_UNROLL; ++u)
      r[u] = __builtin_nontemporal_load(p + at + tid + u * FILTER_THREADS);
  };
  auto fold = [&](const u32x4 (&r)[FILTER_UNROLL]) {
#pragma unroll
    for (uint32_t u = 0; u < FILTER_UNROLL; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  };
  if (b + step <= v1) {
    load(ra, b);
    for (;;) {
      const bool more = b + 2 * step <= v1;
      load(rb, more ? b + step : b);
      fold(ra);
      if (!more) break;
      b += step;
      const bool more2 = b + 2 * step <= v1;
      load(ra, more2 ? b + step : b);
      fold(rb);
      if (!more2) break;
      b += step;
    }
    b += step;
  }
  // the part of the slice after its last whole step
  for (size_t i = b + tid; i < v1; i += FILTER_THREADS) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 63u] = acc;   // keeps the loads
}

hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) cus = 1;
  hipLaunchKernelGGL(k_stream_read, dim3((uint32_t)cus), dim3(FILTER_THREADS), 0, s,
                     static_cast<const u32x4*>(data), bytes / 16, sink);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_finish(const LaunchArgs& a, uint32_t small_k, uint32_t mode,
                                uint32_t bl, uint32_t lk_flags) {
  // one workgroup per compute unit (cached per device)
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = cus > 0 ? cus : 1;
  }
  const Plan& p = a.plan;
  hipLaunchKernelGGL(k_finish<DT>, dim3((uint32_t)cached[dev]), dim3(EX_THREADS), 0, a.stream,
                     a.values, (uint32_t)p.n, (uint32_t)p.rows, a.states, a.rctr, a.call, a.flagged,
                     a.ghist, a.cbuf, a.aux, (uint32_t)p.cap, (uint32_t)p.k, (uint32_t)p.k_eff, p.B,
                     p.W, small_k, mode, a.out_values, a.out_idx, a.lk, bl, lk_flags);
  return hipGetLastError();
}

hipError_t launch_pipeline(const LaunchArgs& a) {
  const Plan& p = a.plan;
  const uint32_t rows = (uint32_t)p.rows, n = (uint32_t)p.n, k = (uint32_t)p.k;
  const bool bucket_sort = !p.small_k && p.cap <= LK_CAP_MAX;
  uint32_t bl = 0;   // index bits that vary: 2^bl >= n
  while (bl < 32 && (1ull << bl) < (uint64_t)n) ++bl;
  bool hist_done = false;
  const uint32_t cap = (uint32_t)p.cap, B = p.B, W = p.W;
  hipStream_t s = a.stream;
  const int dt = p.dtype;
  const dim3 row_grid(rows);
  const dim3 tiny((rows + 63) / 64);
  auto mark = [&](int stage, int begin) {
    if (a.mark) a.mark(a.mark_ctx, stage, begin, s);
  };

  if (p.path == PLAN_EXACT_SMALL) {
    mark(STAGE_EXACT, 1);
    TK_DISPATCH(dt, k_exact_small, row_grid, dim3(SEL_THREADS), 0, s, a.values, n, a.states,
                a.cbuf, cap, k, B, W, (uint32_t)(p.small_k ? 1 : 0), a.out_values, a.out_idx);
    mark(STAGE_EXACT, 0);
  } else {
    if (p.path == PLAN_SAMPLED) {
      const uint32_t sgx = (uint32_t)((p.S + SAMPLE_THREADS - 1) / SAMPLE_THREADS);
      const dim3 sg(sgx, rows);
      // small threshold ranks: select from per-workgroup top-t lists; for
      // t <= 8 and few lists every filter workgroup does that itself
      const bool lists = p.t <= (int64_t)TOPT && (int64_t)sgx * p.t <= p.S;
      const uint32_t ns = lists ? sgx * (uint32_t)p.t : (uint32_t)p.S;   // keys to select from
      const bool in_filter = lists && p.t <= 8 && ns <= 4 * FILTER_THREADS;
      mark(STAGE_SAMPLE, 1);
      TK_DISPATCH(dt, k_sample, sg, dim3(SAMPLE_THREADS), 0, s, a.values, n, (uint32_t)p.S,
                  (uint32_t)p.SP, a.seed, p.half_bits, a.skeys, a.shist, (uint32_t)(lists ? 1 : 0),
                  (uint32_t)p.t, in_filter ? a.states : nullptr, a.rctr);
      mark(STAGE_SAMPLE, 0);
      if (!in_filter) {
        mark(STAGE_TAU, 1);
        hipLaunchKernelGGL(k_tau, row_grid, dim3(SEL_THREADS), 0, s, a.skeys, ns, (uint32_t)p.SP,
                           (uint32_t)p.t, (uint32_t)p.KB, a.shist, (uint32_t)(lists ? 1 : 0),
                           a.states, a.rctr);
        mark(STAGE_TAU, 0);
      }
      const dim3 fg(p.filter_bpr, rows);
      mark(STAGE_FILTER, 1);
      TK_DISPATCH(dt, k_filter, fg, dim3(FILTER_THREADS), 0, s, a.values, n, a.states, a.rctr,
                  a.cbuf, a.aux, cap, B, 1u, a.skeys,
                  in_filter ? ns : 0u, (uint32_t)p.SP, (uint32_t)p.t);
      mark(STAGE_FILTER, 0);
    } else {
      hipLaunchKernelGGL(k_setup_exact, tiny, dim3(64), 0, s, a.states, a.call, a.flagged, rows,
                         k);
    }
    // Check, refine, and the exact route for every failed row: one launch.
    uint32_t mode = FIN_LISTED;
    if (p.path == PLAN_SAMPLED) {
      if (rows <= FIN_SCAN_ROWS) {
        mode = FIN_SCAN;
      } else {
        hipLaunchKernelGGL(k_check, tiny, dim3(64), 0, s, a.states, a.rctr, a.call, a.flagged,
                           rows, k, (uint32_t)p.k_eff, cap);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int stage = p.path == PLAN_SAMPLED ? STAGE_REFINE : STAGE_EXACT;
    mark(stage, 1);
    const uint32_t sk = p.small_k ? 1u : 0u;
    // large k: the first bucket-sort step (histograms) runs inside k_finish
    uint32_t lkf = 0;
    if (bucket_sort) lkf = LK_HIST_EXACT | (p.path == PLAN_SAMPLED ? LK_HIST_SAMPLED : 0u);
    switch (dt) {
      case DT_I32: e = launch_finish<DT_I32>(a, sk, mode, bl, lkf); break;
      case DT_F32: e = launch_finish<DT_F32>(a, sk, mode, bl, lkf); break;
      default: e = launch_finish<DT_BF16>(a, sk, mode, bl, lkf); break;
    }
    hist_done = lkf != 0;
    if (e != hipSuccess) return e;
    mark(stage, 0);
  }
  if (bucket_sort) {
    // every row now holds R in [k, cap] candidates: bucket sort, keep k
    mark(STAGE_SORT, 1);
    const dim3 hg((cap + LK_CHUNK - 1) / LK_CHUNK, rows);
    if (!hist_done)
      hipLaunchKernelGGL(k_lk_hist, hg, dim3(LK_THREADS), 0, s, a.states, a.cbuf, cap, B, bl, a.lk);
    hipLaunchKernelGGL(k_lk_scatter, hg, dim3(LK_THREADS), 0, s, a.states, a.cbuf, a.aux, cap, k,
                       B, bl, a.lk, rows);
    const dim3 sgr((k + LK_WIN - 1) / LK_WIN, rows);
    TK_DISPATCH(dt, k_lk_sort, sgr, dim3(LK_THREADS), 0, s, a.values, n, a.states, a.call, a.aux,
                a.cbuf, cap, k, B, bl, a.lk, rows, a.out_values, a.out_idx);
    mark(STAGE_SORT, 0);
  } else if (!p.small_k) {
    // capacities beyond the bucket sort's: tile sort and pairwise merges
    mark(STAGE_SORT, 1);
    const dim3 tg((cap + SORT_TILE - 1) / SORT_TILE, rows);
    hipLaunchKernelGGL(k_tile_sort, tg, dim3(SEL_THREADS), 0, s, a.states, a.cbuf, cap);
    const dim3 mg((cap + 255) / 256, rows);
    uint64_t* src = a.cbuf;
    uint64_t* dst = a.aux;
    for (uint32_t run = SORT_TILE; run < cap; run <<= 1) {
      hipLaunchKernelGGL(k_merge, mg, dim3(256), 0, s, a.states, src, dst, cap, run);
      uint64_t* t = src;
      src = dst;
      dst = t;
    }
    const dim3 og((k + 255) / 256, rows);
    TK_DISPATCH(dt, k_output, og, dim3(256), 0, s, a.values, n, a.states, src, cap, k, B,
                a.out_values, a.out_idx);
    mark(STAGE_SORT, 0);
  }
  return hipGetLastError();
}

__global__ void k_zero_words(uint32_t* __restrict__ p, size_t nwords) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) p[i] = 0u;
}

__global__ void k_zero_bytes(unsigned char* __restrict__ p, size_t nbytes) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nbytes) p[i] = 0;
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  // the workspace is 256-byte aligned, so whole words first, then the bytes
  const size_t nwords = bytes / 4;
  if (nwords) {
    size_t blocks = (nwords + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero_words, dim3((uint32_t)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(p), nwords);
  }
  const size_t rest = bytes - nwords * 4;
  if (rest) {
    hipLaunchKernelGGL(k_zero_bytes, dim3(1), dim3(64), 0, s,
                       static_cast<unsigned char*>(p) + nwords * 4, rest);
  }
  return hipGetLastError();
}

// ======================================================================
// BatchTopK consumer (Prof-K section 5, "Application: BatchTopK Sparse
// Autoencoders": the batch-global selection keeps the K largest of the
// flattened B x d_dict activations).  The kept activations stay where they
// were and every other entry becomes zero; a mask marks the kept ones.
// Two launches on the caller's stream: a zero fill of the outputs, then one
// thread per winner writes it back.
// ======================================================================
constexpr uint32_t FILL_THREADS = 512;
constexpr uint32_t FILL_UNROLL = 4;

// Zero bytes [0, bytes) of p: the 16-byte aligned middle with nontemporal
// 16-byte stores, one contiguous slice per workgroup (FILL_UNROLL stores per
// lane per step); the unaligned head and tail bytes by workgroup 0.  Swept on
// MI355X over 512 MB followed by a 131072-element scatter: every
// nontemporal shape ends at 103-104 us (as does the runtime's memset), while
// plain stores, faster alone, end at 112-124 us because the fill's dirty L2
// lines are written back before the scatter runs.
__global__ __launch_bounds__(FILL_THREADS) void k_fill_zero(unsigned char* __restrict__ p,
                                                             size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  size_t head = (16u - (a & 15u)) & 15u;
  if (head > bytes) head = bytes;
  const size_t nvec = (bytes - head) / 16;
  const size_t tail0 = head + nvec * 16;
  u32x4* vp = reinterpret_cast<u32x4*>(p + head);
  constexpr size_t step = (size_t)FILL_THREADS * FILL_UNROLL;
  const size_t per = ((nvec + gridDim.x - 1) / gridDim.x + step - 1) / step * step;
  const size_t v0 = (size_t)blockIdx.x * per;
  const size_t v1 = v0 + per < nvec ? v0 + per : nvec;
  const u32x4 z = {0u, 0u, 0u, 0u};
  size_t b = v0;
  for (; b + step <= v1; b += step) {
#pragma unroll
    for (uint32_t u = 0; u < FILL_UNROLL; ++u)
      __builtin_nontemporal_store(z, vp + b + threadIdx.x + u * FILL_THREADS);
  }
  for (size_t i = b + threadIdx.x; i < v1; i += FILL_THREADS) __builtin_nontemporal_store(z, vp + i);
  if (blockIdx.x == 0) {
    if (threadIdx.x < head) p[threadIdx.x] = 0;
    if (threadIdx.x < bytes - tail0) p[tail0 + threadIdx.x] = 0;
  }
}

template <int DT>
__global__ void k_scatter_winners(const void* __restrict__ values, const int64_t* __restrict__ idx,
                                  uint64_t rows, uint64_t k, uint64_t n,
                                  void* __restrict__ out_dense, unsigned char* __restrict__ out_mask) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * k) return;
  const uint64_t r = i / k;
  const int64_t j = idx[i];
  if (j < 0 || (uint64_t)j >= n) return;   // not an index of the row: skipped
  const uint64_t o = r * n + (uint64_t)j;
  if (out_dense) {
    if constexpr (DT == DT_BF16)
      static_cast<uint16_t*>(out_dense)[o] = static_cast<const uint16_t*>(values)[i];
    else
      static_cast<uint32_t*>(out_dense)[o] = static_cast<const uint32_t*>(values)[i];
  }
  if (out_mask) out_mask[o] = 1;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (!bytes) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) cus = 1;
  size_t grid = (size_t)cus * 2;
  const size_t vecs = bytes / 16;
  const size_t want = (vecs + (size_t)FILL_THREADS * FILL_UNROLL - 1) / ((size_t)FILL_THREADS * FILL_UNROLL);
  if (want < grid) grid = want ? want : 1;
  hipLaunchKernelGGL(k_fill_zero, dim3((uint32_t)grid), dim3(FILL_THREADS), 0, s,
                     static_cast<unsigned char*>(p), bytes);
  return hipGetLastError();
}

hipError_t launch_scatter(const void* values, const int64_t* idx, uint64_t rows, uint64_t k,
                          uint64_t n, int dtype, void* out_dense, unsigned char* out_mask,
                          hipStream_t s) {
  const uint64_t es = dtype == DT_BF16 ? 2 : 4;
  hipError_t e = hipSuccess;
  if (out_dense) e = launch_fill_zero(out_dense, rows * n * es, s);
  if (e == hipSuccess && out_mask) e = launch_fill_zero(out_mask, rows * n, s);
  if (e != hipSuccess) return e;
  const uint64_t total = rows * k;
  if (!total) return hipSuccess;
  const dim3 grid((uint32_t)((total + 255) / 256));
  TK_DISPATCH(dtype, k_scatter_winners, grid, dim3(256), 0, s, values, idx, rows, k, n, out_dense,
              out_mask);
  return hipGetLastError();
}

uint32_t filter_threads() { return FILTER_THREADS; }
uint32_t filter_unroll() { return FILTER_UNROLL; }
uint32_t sort_tile() { return SORT_TILE; }

}  // namespace tk
