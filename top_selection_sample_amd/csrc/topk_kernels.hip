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
//                  (k_filter_ahead3: the same with three steps loaded before
//                  tau, for the merge of sorted lists)
//   k_check        many rows: list the rows whose candidate count fails
//   k_setup_exact  rows that start on the exact path
//   k_finish       the check, the refine of every accepted row (small k: select,
//                  sort and write the k winners), and the exact route for the
//                  failed rows, in one persistent launch
//   k_exact_small  small rows: the whole exact selection in one workgroup
//   k_tile_sort / k_merge / k_output   large k: sort all candidates
//   k_lk_chunk / k_lk_sort  large k: bucket sort (chunk step, window sort)
//   k_stream_read  measurement aid: the filter's read pattern alone
//   k_fill_zero / k_scatter_winners   the BatchTopK consumer
//
// The kernels live in parts included below in order (sampler and threshold,
// filter and detection, refinement and the one-workgroup route, the finish
// kernel, the large-k sorts); this file holds the rest and the launchers.
#include <mutex>
#include <type_traits>

#include "topk_device.hpp"
#include "topk_launch.hpp"
#include "topk_select.hpp"

namespace tk {

#include "topk_part_sample.hpp"
#include "topk_part_filter.hpp"
#include "topk_part_refine.hpp"
#include "topk_part_finish.hpp"
#include "topk_part_sort.hpp"

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
  const uint32_t G = (uint32_t)cached[dev];
  // (k_finish derives W and the regions below from B and rows)
  if (p.W != p.B + Dt<DT>::KB) return hipErrorInvalidValue;
  const char* st0 = reinterpret_cast<const char*>(a.states);
  if (reinterpret_cast<const char*>(a.call) != st0 - 256 + ws_off_call((uint32_t)p.rows) ||
      reinterpret_cast<const char*>(a.flagged) != st0 - 256 + ws_off_flag((uint32_t)p.rows) ||
      reinterpret_cast<const char*>(a.ghist) != st0 - 256 + ws_off_ghist((uint32_t)p.rows))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_finish<DT>, dim3(G), dim3(EX_THREADS), 0, a.stream, a.states, a.rctr, a.cbuf, (uint32_t)p.rows, mode, (uint32_t)p.k, (uint32_t)p.k_eff,
                     (uint32_t)p.cap, lk_flags | (small_k ? FIN_SMALL_K : 0u), p.B, G,
                     a.values, (uint32_t)p.n, a.aux, a.out_values,
                     a.out_idx, a.lkc, bl, a.spin_limit);
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
                a.cbuf, cap, k, B, W, (uint32_t)(p.small_k ? 1 : 0), a.out_values, a.out_idx,
                a.call, a.hdr, p.sig);
    mark(STAGE_EXACT, 0);
  } else {
    if (p.path == PLAN_SAMPLED && p.force_tau) {
      // the caller's threshold: no sampler, no threshold select
      mark(STAGE_SAMPLE, 1);
      hipLaunchKernelGGL(k_force_tau, dim3(1, rows), dim3(SAMPLE_THREADS), 0, s, a.states, a.rctr,
                         a.call, a.hdr, p.sig, a.tau_key);
      mark(STAGE_SAMPLE, 0);
      const dim3 fg(p.filter_bpr, rows);
      mark(STAGE_FILTER, 1);
      TK_DISPATCH(dt, k_filter, fg, dim3(FILTER_THREADS), 0, s, a.values, a.skeys, a.states, n,
                  0u, (uint32_t)p.SP, (uint32_t)p.t, fg.x, cap, B, 1u, a.rctr, a.cbuf, a.aux,
                  (WsHeader*)nullptr, p.sig, a.filter_trace, a.trace_wgs);
      mark(STAGE_FILTER, 0);
    } else if (p.path == PLAN_SAMPLED) {
      const uint32_t sgx = (uint32_t)((p.S + SAMPLE_THREADS - 1) / SAMPLE_THREADS);
      const dim3 sg(sgx, rows);
      // small threshold ranks: select from per-workgroup lists, of the t
      // largest keys for t <= TOPT_EXTRACT, else of the TOPT largest, sorted;
      // all of them within the row's S key slots.  With few list keys every
      // filter workgroup selects tau itself.
      const uint32_t len = p.t <= (int64_t)TOPT_EXTRACT ? (uint32_t)p.t : TOPT;
      const bool lists = p.t <= (int64_t)TOPT && (int64_t)sgx * len <= p.S;
      const uint32_t ns = lists ? sgx * len : (uint32_t)p.S;   // keys to select from
      const bool in_filter = lists && ns <= TL_PER * FILTER_THREADS;
      mark(STAGE_SAMPLE, 1);
      TK_DISPATCH(dt, k_sample, sg, dim3(SAMPLE_THREADS), 0, s, a.values, a.seed, a.skeys, n,
                  (uint32_t)p.S, (uint32_t)p.SP, p.half_bits, (uint32_t)(lists ? 1 : 0),
                  (uint32_t)p.t,
                  (uint32_t)((p.t <= 8 && ns <= 4 * FILTER_THREADS)
                                 ? TAU_FILTER_LISTS
                                 : (p.t > (int64_t)TOPT_EXTRACT ? TAU_FILTER_MERGE
                                                                : TAU_FILTER_RADIX)),
                  in_filter ? a.states : nullptr, a.rctr, a.call, a.hdr, a.shist, p.sig);
      mark(STAGE_SAMPLE, 0);
      if (!in_filter) {
        mark(STAGE_TAU, 1);
        hipLaunchKernelGGL(k_tau, row_grid, dim3(SEL_THREADS), 0, s, a.skeys, ns, (uint32_t)p.SP,
                           (uint32_t)p.t, (uint32_t)p.KB, a.shist, (uint32_t)(lists ? 1 : 0),
                           a.states, a.rctr, (const WsHeader*)a.hdr, p.sig);
        mark(STAGE_TAU, 0);
      }
      const dim3 fg(p.filter_bpr, rows);
      mark(STAGE_FILTER, 1);
      // after k_tau (all keys) every row's sample histogram is zero again
      WsHeader* validate = lists ? nullptr : a.hdr;
      // (the merge of sorted lists selects tau last: a third step of the
      // stream is loaded before it)
      if (in_filter && p.t > (int64_t)TOPT_EXTRACT) {
        TK_DISPATCH(dt, k_filter_ahead3, fg, dim3(FILTER_THREADS), 0, s, a.values, a.skeys,
                    a.states, n, ns, (uint32_t)p.SP, (uint32_t)p.t, fg.x, cap, B, 1u, a.rctr,
                    a.cbuf, a.aux, validate, p.sig, a.filter_trace, a.trace_wgs);
      } else {
        TK_DISPATCH(dt, k_filter, fg, dim3(FILTER_THREADS), 0, s, a.values, a.skeys, a.states, n,
                    in_filter ? ns : 0u, (uint32_t)p.SP, (uint32_t)p.t, fg.x, cap, B, 1u,
                    a.rctr, a.cbuf, a.aux, validate, p.sig, a.filter_trace, a.trace_wgs);
      }
      mark(STAGE_FILTER, 0);
    } else {
      hipLaunchKernelGGL(k_setup_exact, tiny, dim3(64), 0, s, a.states, a.call, a.flagged, rows,
                         k, a.hdr, p.sig);
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
      hipLaunchKernelGGL(k_lk_chunk, hg, dim3(LK_THREADS), 0, s, a.states, a.cbuf, cap, B, bl,
                         a.lkc);
    const dim3 sgr((k + LK_WIN - 1) / LK_WIN, rows);
    TK_DISPATCH(dt, k_lk_sort, sgr, dim3(LK_THREADS), 0, s, a.values, n, a.states, a.call, a.cbuf,
                a.aux, a.lks, cap, k, B, bl, a.lkc, a.out_values, a.out_idx);
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

// ======================================================================
// Built-in scratch for callers that cannot allocate (topk_noalloc): a
// file-scope device array, one per GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: its
// device address is looked up once per device (with that device current)
// and kept.
// ======================================================================
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

uint32_t filter_threads() { return FILTER_THREADS; }
uint32_t filter_unroll() { return FILTER_UNROLL; }
uint32_t sort_tile() { return SORT_TILE; }

}  // namespace tk
