// Internal interface between the host dispatcher and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tk {

struct RowState;
struct RowCtr;
struct CallState;
struct WsHeader;

enum : int { PLAN_SAMPLED = 0, PLAN_EXACT = 1, PLAN_EXACT_SMALL = 2 };

constexpr int64_t KSMALL = 4096;            // largest k sorted inside one workgroup
constexpr int64_t LK_CAP_MAX = int64_t(1) << 21;  // large k: bucket sort up to this capacity
constexpr uint32_t LK_RANKS = 4096;         // large k: buckets of the bucket sort
constexpr uint32_t LK_CSTRIDE = 4096 + 64;   // words per chunk: prefix counts, then every 64th
constexpr int64_t LK_CHUNK_CANDS = 4096;    // candidates per chunk of the bucket sort
constexpr int64_t EXACT_SMALL_MAX = 1 << 18; // rows this short run in one workgroup

struct Plan {
  int64_t n = 0, rows = 0, k = 0;
  int64_t k_eff = 0;   // k, or ceil(recall * k) in relaxed-recall mode
  int dtype = 0;
  int path = PLAN_SAMPLED;
  bool small_k = true;
  int64_t S = 0, SP = 0, t = 0, M = 0, cap = 0;
  uint32_t B = 8, W = 40, KB = 32, half_bits = 1;
  uint32_t filter_bpr = 1, hist_bpr = 1;
  double p_recall = 0, p_overflow = 0;
  bool force_tau = false;   // the caller gives the threshold: no sampler
  // workspace layout (byte offsets; the header is at 0)
  uint64_t sig = 0;         // layout signature (never 0)
  size_t off_states = 0, off_call = 0, off_flag = 0, off_ghist = 0, off_skeys = 0, off_shist = 0, off_cbuf = 0, off_aux = 0, off_lkc = 0, off_lks = 0, off_rctr = 0, total = 0;
};

// Pipeline stages that can be bracketed by timing events.
enum : int { STAGE_SAMPLE = 0, STAGE_TAU = 1, STAGE_FILTER = 2, STAGE_REFINE = 3,
             STAGE_EXACT = 4, STAGE_SORT = 5, STAGE_COUNT = 6 };

// Called before (begin = 1) and after (begin = 0) a stage's launches.
typedef void (*StageMark)(void* ctx, int stage, int begin, hipStream_t s);

// Test aid (topk_params.test_flags): every grid-barrier wait of the exact
// route gives up at once.
constexpr uint32_t TEST_BARRIER_GIVEUP = 1u;
constexpr uint32_t SPIN_LIMIT_DEFAULT = 1u << 22;   // polls before a barrier wait gives up

struct LaunchArgs {
  StageMark mark = nullptr;
  void* mark_ctx = nullptr;
  Plan plan;
  WsHeader* hdr;
  uint32_t tau_key = 0;          // plan.force_tau: the threshold key of every row
  uint32_t spin_limit = SPIN_LIMIT_DEFAULT;
  uint64_t* filter_trace = nullptr;   // measurement aid: per-workgroup stamps of the filter
  uint32_t trace_wgs = 0;             //   (for workgroups below this count)
  const void* values;
  void* out_values;
  int64_t* out_idx;
  RowState* states;
  RowCtr* rctr;      // sampled route: per-row filter counters
  CallState* call;
  uint32_t* flagged;
  uint32_t* ghist;
  uint32_t* skeys;
  uint32_t* shist;
  uint64_t* cbuf;
  uint64_t* aux;     // large k: merge buffer; sampled route: tie region (rows x cap)
  uint32_t* lkc;     // large-k bucket sort: per chunk, its prefix count by rank
  uint64_t* lks;     // large-k bucket sort: split scratch (rows x cap)
  uint64_t seed;
  hipStream_t stream;
};

// Bytes of the built-in scratch array of topk_noalloc (per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(32) << 20;
// Its device address on the current device (looked up on the first call per
// device, then kept).
hipError_t noalloc_scratch(void** out);

hipError_t launch_pipeline(const LaunchArgs& a);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);
hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_scatter(const void* values, const int64_t* idx, uint64_t rows, uint64_t k,
                          uint64_t n, int dtype, void* out_dense, unsigned char* out_mask,
                          hipStream_t s);
uint32_t filter_threads();
uint32_t filter_unroll();
uint32_t sort_tile();

}  // namespace tk
