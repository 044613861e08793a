// Device-side building blocks of the exact top-k engine (gfx950, wave64).
//
// Order used everywhere: an element outranks another when its value is
// larger, or when the values are equal and its index is lower (GPU.js Learn,
// "Rank by Counting", Goal).  Values are compared through order-preserving
// unsigned keys; an element is then identified by its composite
//
//     comp = key << B | (2^B - 1 - index)          (B = index bits, mult. of 8)
//
// which is unique per element and orders exactly as the rank does, so "the k
// largest composites" is the answer, ties included.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tk {

enum : int { DT_I32 = 0, DT_F32 = 1, DT_BF16 = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Per-row phase of the pipeline.
enum : uint32_t {
  ST_IDLE = 0,
  ST_FILTER = 1,       // sampled threshold set; sampled filter pass pending/done
  ST_EXACT = 2,        // exact radix select over the whole row in progress
  ST_EXACT_READY = 3,  // exact threshold known; exact filter pass pending/done
  ST_SORT = 4,         // candidates ready for the multi-workgroup sort
  ST_DONE = 5,
};

// Which route produced a row's answer (reported through the stats call).
enum : uint32_t { PATH_SAMPLED = 0, PATH_FALLBACK = 1, PATH_EXACT = 2, PATH_PARTIAL = 3 };

struct alignas(64) RowState {
  uint32_t status;
  uint32_t tau_key;     // sampled threshold key (t-th largest sampled key)
  uint32_t count;       // candidates counted by the current filter pass (sampled
                        //   pass: elements strictly above tau)
  uint32_t ties;        // sampled pass: elements equal to tau (published copy)
  uint32_t r_sampled;   // survivors of the sampled pass
  uint32_t path;        // PATH_*
  uint32_t need;        // exact select: rank wanted inside the prefix bucket
  uint32_t above;       // exact select: elements above the prefix bucket
  uint64_t prefix;      // exact select: resolved top bits of the composite
  uint32_t nbits;       // exact select: number of resolved bits
  uint32_t thr_key;     // exact threshold: key >= thr_key, and on key ==
  uint32_t thr_bound;   //   thr_key only indices <= thr_bound
  uint32_t passes;      // exact select: histogram passes used
  uint32_t tau_route;   // how the threshold was selected (TAU_* bits, a diagnostic)
  uint32_t kmax;        // largest candidate key written by a filter pass
};
static_assert(sizeof(RowState) == 64, "RowState is one 64-byte line");

// Counters that every filter workgroup updates once at its end, each on a
// 128-byte line of its own: atomics on one line serialise, and four of them
// per workgroup on the row's state line measured about 12 us slower over
// 512 workgroups than one.
struct alignas(128) RowCtr {
  uint32_t ties;        // elements equal to tau (exact count)
  uint32_t pad0[31];
  uint32_t tslots;      // tie-region slots claimed
  uint32_t pad1[31];
  uint32_t kmax;        // largest key above tau
  uint32_t pad2[31];
  uint32_t above;       // elements above tau (a count the finish kernel never rewrites)
  uint32_t pad3[31];
};
static_assert(sizeof(RowCtr) == 512, "four 128-byte lines");

// How a row's threshold was selected (RowState::tau_route): the source in
// the low bits, and whether the boundary bin of the sample histogram held
// more keys than LDS (streamed radix select) or more than the rank-counting
// limit (radix select in LDS).
enum : uint32_t {
  TAU_NONE = 0,          // no sampled threshold (exact route)
  TAU_FILTER_LISTS = 1,  // per-workgroup top-t lists, selected in the filter's prologue
  TAU_KTAU_LISTS = 2,    // per-workgroup top-t lists, selected by k_tau
  TAU_KTAU_REGS = 3,     // every sample key, held in k_tau's registers
  TAU_KTAU_STREAM = 4,   // every sample key, streamed by k_tau
  TAU_FORCED = 5,        // given by the caller
  TAU_FILTER_RADIX = 6,  // per-workgroup top-t lists, radix-selected in the filter's prologue
  TAU_FILTER_MERGE = 7,  // per-workgroup sorted lists of 32, merged in the filter's prologue
  TAU_BIN_STREAMED = 8,  // flag: the boundary bin exceeded LDS
  TAU_BIN_RADIX = 16,    // flag: the boundary bin was radix-selected in LDS
};

// Per-call record shared by all rows: the rows sent to the exact route and
// the exact route's grid-barrier words.  The first kernel of every call
// writes it to zero; nothing is carried from one call to the next.
struct alignas(64) CallState {
  uint32_t nflag;      // rows listed for the exact route
  uint32_t nactive;    // listed rows whose exact threshold is not resolved yet
  uint32_t bar_count;  // grid barrier: arrivals in the current round
  uint32_t bar_gen;    // grid barrier: round number
  uint32_t error;      // bit 0: a grid-barrier wait gave up (the listed rows were
                       //   then selected again by one workgroup); bit 1: the
                       //   large-k sort's pending-range stack overflowed
  uint32_t exit_count; // exact route: workgroups that have finished it
  uint32_t pad[10];
};
static_assert(sizeof(CallState) == 64, "CallState is one 64-byte line");

__device__ __forceinline__ void reset_call(CallState* cs) {
  cs->nflag = 0;
  cs->nactive = 0;
  cs->bar_count = 0;
  cs->bar_gen = 0;
  cs->error = 0;
  cs->exit_count = 0;
}

// Workspace header (its first 256 bytes).  `stamp` is the layout signature
// of the call whose sample-histogram region is known to be all zero, or 0:
// a call uses that region only when the stamp is its own signature, and
// leaves it zero and stamped when it has used it.  Every other region is
// written before it is read within a call, so a workspace needs no
// initialisation and may hold anything between calls.
struct alignas(256) WsHeader {
  uint64_t stamp;
  uint64_t pad[31];
};
static_assert(sizeof(WsHeader) == 256, "one 256-byte header");

// A call that will not validate the stamp (any call whose layout differs,
// and every call that does not build the sample histogram) clears it unless
// it is already its own: the call may overwrite the region.  Racing readers
// in the same kernel see either value, and neither equals `sig`.
// The workspace's first regions follow from the row count alone (the header,
// the row states, the call record, the flagged-row list and the exact-route
// histograms, each 256-byte aligned), so a kernel that has the row states
// finds the rest without arguments that would have to be loaded.
__host__ __device__ __forceinline__ size_t ws_align256(size_t v) { return (v + 255) & ~(size_t)255; }
__host__ __device__ __forceinline__ size_t ws_off_call(uint32_t rows) {
  return ws_align256(256 + (size_t)rows * 64);
}
__host__ __device__ __forceinline__ size_t ws_off_flag(uint32_t rows) {
  return ws_align256(ws_off_call(rows) + 64);
}
__host__ __device__ __forceinline__ size_t ws_off_ghist(uint32_t rows) {
  return ws_align256(ws_off_flag(rows) + (size_t)rows * 4);
}
// (the row states start at byte 256)
template <class T>
__device__ __forceinline__ T* ws_region(const void* states, size_t off) {
  return reinterpret_cast<T*>(const_cast<char*>(static_cast<const char*>(states)) - 256 + off);
}

// The workgroup size a kernel is always launched with, told to the compiler:
// blockDim.x is otherwise read from the dispatch's hidden arguments, a memory
// round trip at the start of the kernel.
#define assume_block_threads(N)                   \
  do {                                            \
    const uint32_t bd_ = blockDim.x;              \
    __builtin_assume(bd_ == (uint32_t)(N));       \
  } while (0)

__device__ __forceinline__ void stamp_invalidate(WsHeader* h, uint64_t sig) {
  if (h->stamp != sig) h->stamp = 0;
}

// ---------------------------------------------------------------- keys
// int32: flip the sign bit.  float (32 or 16 bit): a negative value flips all
// bits, a positive one sets the sign bit; -0 maps to +0's key and every NaN to
// the top key, so NaN ranks above +inf and ties with other NaNs by index.
__device__ __forceinline__ uint32_t key_i32(uint32_t b) { return b ^ 0x80000000u; }

__device__ __forceinline__ uint32_t key_f32(uint32_t b) {
  uint32_t flip = (uint32_t)((int32_t)b >> 31) | 0x80000000u;
  uint32_t k = b ^ flip;
  uint32_t mag = b & 0x7FFFFFFFu;
  k = (mag == 0u) ? 0x80000000u : k;
  k = (mag > 0x7F800000u) ? 0xFFFFFFFFu : k;
  return k;
}

__device__ __forceinline__ uint32_t key_bf16(uint32_t h) {  // h: 16 bits
  uint32_t flip = ((h & 0x8000u) ? 0xFFFFu : 0x8000u);
  uint32_t k = h ^ flip;
  uint32_t mag = h & 0x7FFFu;
  k = (mag == 0u) ? 0x8000u : k;
  k = (mag > 0x7F80u) ? 0xFFFFu : k;
  return k;
}

// Inverse of the key for every key except the two that several bit patterns
// share: +0's key (also -0) and the top key (every NaN).  Returns false for
// those; the caller then reads the element itself.
__device__ __forceinline__ bool unkey_f32(uint32_t k, uint32_t* bits) {
  if (k == 0x80000000u || k == 0xFFFFFFFFu) return false;
  *bits = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return true;
}
__device__ __forceinline__ bool unkey_bf16(uint32_t k, uint32_t* bits) {
  if (k == 0x8000u || k == 0xFFFFu) return false;
  *bits = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return true;
}

template <int DT> struct Dt;
template <> struct Dt<DT_I32> {
  using raw = uint32_t;
  static constexpr int KB = 32;      // key bits
  static constexpr int ES = 4;       // element bytes
  static constexpr int VEC = 4;      // elements per 16-byte load
  __device__ static uint32_t key(uint32_t r) { return key_i32(r); }
  __device__ static bool unkey(uint32_t k, uint32_t* bits) {
    *bits = k ^ 0x80000000u;
    return true;
  }
};
template <> struct Dt<DT_F32> {
  using raw = uint32_t;
  static constexpr int KB = 32, ES = 4, VEC = 4;
  __device__ static uint32_t key(uint32_t r) { return key_f32(r); }
  __device__ static bool unkey(uint32_t k, uint32_t* bits) { return unkey_f32(k, bits); }
};
template <> struct Dt<DT_BF16> {
  using raw = uint16_t;
  static constexpr int KB = 16, ES = 2, VEC = 8;
  __device__ static uint32_t key(uint32_t r) { return key_bf16(r & 0xFFFFu); }
  __device__ static bool unkey(uint32_t k, uint32_t* bits) { return unkey_bf16(k, bits); }
};

// Raw bits of element i of a row.
template <int DT>
__device__ __forceinline__ uint32_t load_raw(const void* row, uint32_t i) {
  if constexpr (DT == DT_BF16) {
    return static_cast<const uint16_t*>(row)[i];
  } else {
    return static_cast<const uint32_t*>(row)[i];
  }
}

__device__ __forceinline__ uint64_t make_comp(uint32_t key, uint32_t idx, uint32_t B) {
  uint64_t maskB = (B >= 64) ? ~0ull : ((1ull << B) - 1ull);
  return ((uint64_t)key << B) | (maskB - (uint64_t)idx);
}

__device__ __forceinline__ uint32_t comp_index(uint64_t c, uint32_t B) {
  uint64_t maskB = (1ull << B) - 1ull;
  return (uint32_t)(maskB - (c & maskB));
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ uint32_t rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// A uniform lane's value, read into a scalar register.
__device__ __forceinline__ uint32_t wave_bcast(uint32_t v, uint32_t lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)lane);
}

// Inclusive scans over the 64 lanes of a wave with DPP moves: shifts by 1,
// 2, 4 and 8 lanes inside each row of 16, then lane 15 of each row into the
// next row and lane 31 into the upper half.  A lane whose source is outside
// its row (or whose row is masked off) takes the identity 0.  Every lane of
// the wave must be active: the moves read the other lanes' registers, so
// each one is taken into a temporary before it is combined (a combine that
// re-reads it could be turned into a branch with lanes switched off).  The
// result leaves through an empty asm: without it the compiler may fold the
// caller's arithmetic into the last move (a row-broadcast subtract,
// v_subrev_u32_dpp row_bcast:31, which gave wrong sums on gfx950 where the
// move-then-add form is right).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_take(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  uint32_t t;
  t = dpp_take<0x111, 0xf>(v); v += t;
  t = dpp_take<0x112, 0xf>(v); v += t;
  t = dpp_take<0x114, 0xf>(v); v += t;
  t = dpp_take<0x118, 0xf>(v); v += t;
  t = dpp_take<0x142, 0xa>(v); v += t;
  t = dpp_take<0x143, 0xc>(v); v += t;
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
  uint32_t t;
  t = dpp_take<0x111, 0xf>(v); v = __builtin_elementwise_max(v, t);
  t = dpp_take<0x112, 0xf>(v); v = __builtin_elementwise_max(v, t);
  t = dpp_take<0x114, 0xf>(v); v = __builtin_elementwise_max(v, t);
  t = dpp_take<0x118, 0xf>(v); v = __builtin_elementwise_max(v, t);
  t = dpp_take<0x142, 0xa>(v); v = __builtin_elementwise_max(v, t);
  t = dpp_take<0x143, 0xc>(v); v = __builtin_elementwise_max(v, t);
  asm volatile("" : "+v"(v));
  return v;
}

// 64-bit minimum and maximum over the wave, uniform: the same scan on both
// halves of each value (identity ~0 for the minimum, 0 for the maximum).
template <int CTRL, int ROWS, int ID>
__device__ __forceinline__ uint64_t dpp_take64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t bcast64(uint64_t v, uint32_t lane) {
  return ((uint64_t)wave_bcast((uint32_t)(v >> 32), lane) << 32) | wave_bcast((uint32_t)v, lane);
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  uint64_t t;
  t = dpp_take64<0x111, 0xf, -1>(v); v = t < v ? t : v;
  t = dpp_take64<0x112, 0xf, -1>(v); v = t < v ? t : v;
  t = dpp_take64<0x114, 0xf, -1>(v); v = t < v ? t : v;
  t = dpp_take64<0x118, 0xf, -1>(v); v = t < v ? t : v;
  t = dpp_take64<0x142, 0xa, -1>(v); v = t < v ? t : v;
  t = dpp_take64<0x143, 0xc, -1>(v); v = t < v ? t : v;
  return bcast64(v, 63u);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t t;
  t = dpp_take64<0x111, 0xf, 0>(v); v = t > v ? t : v;
  t = dpp_take64<0x112, 0xf, 0>(v); v = t > v ? t : v;
  t = dpp_take64<0x114, 0xf, 0>(v); v = t > v ? t : v;
  t = dpp_take64<0x118, 0xf, 0>(v); v = t > v ? t : v;
  t = dpp_take64<0x142, 0xa, 0>(v); v = t > v ? t : v;
  t = dpp_take64<0x143, 0xc, 0>(v); v = t > v ? t : v;
  return bcast64(v, 63u);
}

// Sum and maximum over the wave, uniform (lane 63's inclusive scan).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_bcast(wave_incl_sum(v), 63u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_bcast(wave_incl_max(v), 63u);
}

// Orders this wave's earlier LDS accesses before its later ones, as seen by
// the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- buckets
// Find, over a 256-bin histogram ordered from bin 255 (largest digit) down,
// the bin b holding the element of rank `need` (1-based from the top), and
// `acc` = number of elements in bins above b.  Run by the 64 lanes of one
// wave; the result lands in out[0] = b, out[1] = acc, out[2] = hist[b].
__device__ __forceinline__ void wave_find_bucket(const uint32_t* hist, uint32_t need,
                                                 uint32_t* out) {
  const uint32_t l = lane_id();
  const uint32_t b3 = 255u - 4u * l;
  uint32_t c3 = hist[b3], c2 = hist[b3 - 1], c1 = hist[b3 - 2], c0 = hist[b3 - 3];
  uint32_t s = c3 + c2 + c1 + c0;
  const uint32_t incl = wave_incl_sum(s);
  uint64_t m = ballot(incl >= need);
  uint32_t first = m ? (uint32_t)__builtin_ctzll(m) : 63u;
  if (l == first) {
    uint32_t acc = incl - s, b, hb;
    if (acc + c3 >= need) { b = b3; hb = c3; }
    else if (acc + c3 + c2 >= need) { acc += c3; b = b3 - 1; hb = c2; }
    else if (acc + c3 + c2 + c1 >= need) { acc += c3 + c2; b = b3 - 2; hb = c1; }
    else { acc += c3 + c2 + c1; b = b3 - 3; hb = c0; }
    out[0] = b;
    out[1] = acc;
    out[2] = hb;
  }
}

// The same over a 2048-bin histogram by a whole workgroup of NT threads
// (every thread calls it; the result is in out[] after the caller's next
// barrier): thread i holds bins [2048 i / NT, 2048 (i + 1) / NT), each wave
// posts its total to s_wt (NT / 64 words), and the one thread whose bins
// hold the rank resolves it.  Four dependent LDS and DPP steps per thread
// instead of one wave walking all 2048 bins.  Needs 1 <= need <= the total.
template <uint32_t NT>
__device__ __forceinline__ void block_find_bucket_2048(const uint32_t* hist, uint32_t need,
                                                       uint32_t* out, uint32_t* s_wt) {
  constexpr uint32_t BPT = 2048 / NT, NW = NT / 64;
  static_assert(BPT * NT == 2048 && (BPT == 2 || BPT == 4), "2 or 4 bins per thread");
  const uint32_t tid = threadIdx.x, l = tid & 63u, w = tid >> 6;
  uint32_t h[BPT];
  if constexpr (BPT == 2) {
    const uint2 v = reinterpret_cast<const uint2*>(hist)[tid];
    h[0] = v.x;
    h[1] = v.y;
  } else {
    const uint4 v = reinterpret_cast<const uint4*>(hist)[tid];
    h[0] = v.x;
    h[1] = v.y;
    h[2] = v.z;
    h[3] = v.w;
  }
  uint32_t mine = 0;
#pragma unroll
  for (uint32_t q = 0; q < BPT; ++q) mine += h[q];
  const uint32_t incl = wave_incl_sum(mine);
  const uint32_t wtot = wave_bcast(incl, 63u);
  if (l == 0) s_wt[w] = wtot;
  __syncthreads();
  uint32_t above = 0;   // elements in the waves holding higher bins
#pragma unroll
  for (uint32_t q = 0; q < NW; ++q) above += q > w ? s_wt[q] : 0u;
  above += wtot - incl;   // ... and in this wave's higher lanes
  if (above < need && above + mine >= need) {
    uint32_t a = above, b = BPT * tid, hb = h[0];
    bool found = false;
#pragma unroll
    for (int q = (int)BPT - 1; q >= 0; --q) {
      if (!found && a + h[q] >= need) {
        found = true;
        b = BPT * tid + (uint32_t)q;
        hb = h[q];
      } else if (!found) {
        a += h[q];
      }
    }
    out[0] = b;
    out[1] = a;
    out[2] = hb;
  }
}

// The same over a 2048-bin histogram.  Read step j gives lane l the four
// bins 256j + 4l .. 256j + 4l + 3 (consecutive lanes read consecutive 16-byte
// words: no bank conflicts).  The group of 256 bins holding the rank is
// found from the group totals, then the lane inside it from a suffix sum
// over the lanes (higher lanes hold higher bins).
__device__ __forceinline__ void wave_find_bucket_2048(const uint32_t* hist, uint32_t need,
                                                      uint32_t* out) {
  const uint32_t l = lane_id();
  const uint4* hp = reinterpret_cast<const uint4*>(hist);
  uint32_t s[8], tot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 h = hp[64 * j + l];
    s[j] = h.x + h.y + h.z + h.w;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) tot[j] = wave_sum_u32(s[j]);
  // the group, from the top (uniform)
  uint32_t acc = 0, g = 0;
  bool gfound = false;
#pragma unroll
  for (int j = 7; j >= 0; --j) {
    if (!gfound && acc + tot[j] >= need) {
      gfound = true;
      g = (uint32_t)j;
    } else if (!gfound) {
      acc += tot[j];
    }
  }
  uint32_t sg = s[0], tg = tot[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    if (g == (uint32_t)j) {
      sg = s[j];
      tg = tot[j];
    }
  }
  const uint4 hg = hp[64 * g + l];   // the group's four bins, read again
  // elements in this lane's bins and every higher lane's, within the group
  const uint32_t suffix = tg - wave_incl_sum(sg) + sg;
  const uint64_t m = ballot(acc + suffix >= need);
  const uint32_t lf = m ? 63u - (uint32_t)__builtin_clzll(m) : 0u;
  if (l == lf) {
    uint32_t a = acc + suffix - sg, b = 256u * g + 4u * l, hb = hg.x;
    const uint32_t v[4] = {hg.w, hg.z, hg.y, hg.x};
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!found && a + v[q] >= need) {
        found = true;
        b = 256u * g + 4u * l + 3u - (uint32_t)q;
        hb = v[q];
      } else if (!found) {
        a += v[q];
      }
    }
    out[0] = b;
    out[1] = a;
    out[2] = hb;
  }
}

}  // namespace tk
