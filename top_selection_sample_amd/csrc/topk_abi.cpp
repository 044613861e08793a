// C ABI entry points of the exact top-k library: argument checks, the plan
// of the call shape, workspace carving and the launch of the pipeline.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/topk.h"
#include "topk_device.hpp"
#include "topk_launch.hpp"
#include "topk_plan.hpp"

namespace {

std::atomic<uint64_t> g_calls{0};

// ---- filter workgroup trace (measurement aid)
std::atomic<uint64_t*> g_trace_buf{nullptr};
std::atomic<uint64_t> g_trace_words{0};

// ---- stage timing
std::atomic<int> g_prof{0};
std::mutex g_prof_mu;
struct Bracket {
  hipEvent_t a, b;
  int stage;
};
std::vector<Bracket> g_done;                  // closed brackets
hipEvent_t g_open[tk::STAGE_COUNT] = {};       // begin events awaiting their end
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void mark_stage(void*, int stage, int begin, hipStream_t s) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    g_pool.push_back(e);
    return;
  }
  if (begin) {
    if (g_open[stage]) g_pool.push_back(g_open[stage]);
    g_open[stage] = e;
  } else if (g_open[stage]) {
    g_done.push_back(Bracket{g_open[stage], e, stage});
    g_open[stage] = nullptr;
  } else {
    g_pool.push_back(e);
  }
}

tk::ParamIn to_in(const topk_params* p) {
  tk::ParamIn in;
  if (!p) return in;
  in.eps = p->eps;
  in.s_min = p->s_min;
  in.s_max = p->s_max;
  in.cost_ratio = p->cost_ratio;
  in.policy = p->policy;
  in.force_path = p->force_path;
  in.S = p->S;
  in.t = p->t;
  in.M = p->M;
  in.tuned_ratio = p->tuned_ratio;
  in.tuned_s_min = p->tuned_s_min;
  in.tuned_ratio_large = p->tuned_ratio_large;
  in.tuned_ratio_batched = p->tuned_ratio_batched;
  in.tuned_batch_rows = p->tuned_batch_rows;
  in.recall = p->recall;
  in.force_tau = p->use_force_tau != 0;
  return in;
}

int check_params(const topk_params* p) {
  if (!p) return TOPK_OK;
  if (!(p->eps > 0.0 && p->eps < 1.0)) return TOPK_EINVAL;
  if (p->s_min < 1 || p->s_max < p->s_min) return TOPK_EINVAL;
  if (!(p->cost_ratio > 0.0)) return TOPK_EINVAL;
  if (p->policy < 0 || p->policy > 2) return TOPK_EINVAL;
  if (!(p->tuned_ratio > 0.0) || p->tuned_s_min < 1) return TOPK_EINVAL;
  if (!(p->tuned_ratio_large > 0.0)) return TOPK_EINVAL;
  if (!(p->tuned_ratio_batched > 0.0) || p->tuned_batch_rows < 1) return TOPK_EINVAL;
  if (!(p->recall > 0.0 && p->recall <= 1.0)) return TOPK_EINVAL;
  if (p->force_path < 0 || p->force_path > 2) return TOPK_EINVAL;
  if (p->S < 0 || p->t < 0 || p->M < 0) return TOPK_EINVAL;
  if (p->use_force_tau && p->force_path == TOPK_PATH_EXACT) return TOPK_EINVAL;
  if (p->test_flags & ~(uint32_t)TOPK_TEST_BARRIER_GIVEUP) return TOPK_EINVAL;
  return TOPK_OK;
}

int check_shape(int64_t n, int64_t rows, int64_t k, int dtype) {
  if (dtype < 0 || dtype > 2) return TOPK_EDTYPE;
  if (n < 1 || rows < 1 || k < 1 || k > n) return TOPK_EINVAL;
  if (n > (int64_t)0xFFFFFFFEll) return TOPK_EINVAL;   // indices stay below 2^32 - 1
  if (rows > 65535) return TOPK_EINVAL;                 // rows ride on grid dimension y
  return TOPK_OK;
}

// Compute units of the current device (cached per device; 256 when no
// device is present, e.g. for a plan query on a host without a GPU).
int64_t device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int plan_of(int64_t n, int64_t rows, int64_t k, int dtype, const topk_params* params,
            tk::Plan* plan, bool with_device) {
  int rc = check_shape(n, rows, k, dtype);
  if (rc) return rc;
  rc = check_params(params);
  if (rc) return rc;
  tk::ParamIn in = to_in(params);
  in.cus = with_device ? device_cus() : 256;
  if (in.force_path == 1 && n < 2) return TOPK_EINVAL;
  tk::make_plan(n, rows, k, dtype, in, plan);
  if (plan->path == tk::PLAN_SAMPLED && (plan->S < 1 || plan->S > n || plan->t < 1 || plan->t > plan->S))
    return TOPK_EINVAL;
  return TOPK_OK;
}

}  // namespace

extern "C" {

static_assert(sizeof(topk_params) == 136, "topk_params layout is part of the ABI");
static_assert(sizeof(topk_row_stats) == 28, "topk_row_stats layout is part of the ABI");
static_assert(sizeof(tk::WsHeader) == 256 && sizeof(tk::RowState) == 64, "workspace header and rows");

int topk_default_params(topk_params* p) {
  if (!p) return TOPK_EINVAL;
  std::memset(p, 0, sizeof(*p));
  p->eps = 1e-3;
  p->s_min = 32768;
  p->s_max = 131072;
  p->cost_ratio = 1.0;
  p->policy = TOPK_POLICY_TUNED;
  p->force_path = TOPK_PATH_AUTO;
  p->tuned_ratio = 0.13;
  p->tuned_s_min = 1024;
  p->tuned_ratio_large = 0.01;
  p->tuned_ratio_batched = 0.03;
  p->tuned_batch_rows = 32;
  p->recall = 1.0;
  return TOPK_OK;
}

int topk_plan(int64_t n, int64_t rows, int64_t k, int dtype, const topk_params* params,
              topk_plan_info* out) {
  if (!out) return TOPK_EINVAL;
  try {
    tk::Plan p;
    int rc = plan_of(n, rows, k, dtype, params, &p, false);
    if (rc) return rc;
    out->path = p.path;
    out->small_k = p.small_k ? 1 : 0;
    out->S = p.S;
    out->t = p.t;
    out->M = p.M;
    out->cap = p.cap;
    out->index_bits = (int32_t)p.B;
    out->key_bits = (int32_t)p.KB;
    out->k_eff = p.k_eff;
    out->p_recall = p.p_recall;
    out->p_overflow = p.p_overflow;
    out->workspace_bytes = p.total;
    return TOPK_OK;
  } catch (...) {
    return TOPK_EINVAL;
  }
}

int topk_workspace_size(int64_t n, int64_t rows, int64_t k, int dtype, const topk_params* params,
                        size_t* bytes) {
  if (!bytes) return TOPK_EINVAL;
  topk_plan_info info;
  int rc = topk_plan(n, rows, k, dtype, params, &info);
  if (rc) return rc;
  *bytes = info.workspace_bytes;
  return TOPK_OK;
}

int topk_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace && bytes) return TOPK_EINVAL;
  if (!bytes) return TOPK_OK;
  hipError_t e = tk::launch_zero_fill(workspace, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TOPK_OK : TOPK_EHIP;
}

}  // extern "C"

namespace {

// The body of topk_ex.  allow_marks = false: no stage-timing events (they
// are created on demand), for topk_noalloc.
int topk_run(const void* values, int64_t n, int64_t rows, int64_t k, int dtype, void* out_values,
             int64_t* out_indices, void* workspace, size_t workspace_bytes, void* stream,
             const topk_params* params, bool allow_marks) {
  if (!values || !out_values || !out_indices || !workspace) return TOPK_EINVAL;
  try {
    tk::Plan p;
    int rc = plan_of(n, rows, k, dtype, params, &p, true);
    if (rc) return rc;
    const uintptr_t es = (dtype == TOPK_BF16) ? 2 : 4;
    if (reinterpret_cast<uintptr_t>(values) % es || reinterpret_cast<uintptr_t>(out_values) % es ||
        reinterpret_cast<uintptr_t>(out_indices) % 8 || reinterpret_cast<uintptr_t>(workspace) % 256)
      return TOPK_EINVAL;
    if (workspace_bytes < p.total) return TOPK_EWORKSPACE;
    char* ws = static_cast<char*>(workspace);
    tk::LaunchArgs a;
    a.plan = p;
    a.hdr = reinterpret_cast<tk::WsHeader*>(ws);
    a.tau_key = (params && params->use_force_tau) ? params->force_tau_key : 0u;
    if (params && (params->test_flags & TOPK_TEST_BARRIER_GIVEUP)) a.spin_limit = 0;
    a.filter_trace = g_trace_buf.load();
    {
      const uint64_t wgs = g_trace_words.load() / 2;
      a.trace_wgs = a.filter_trace ? (uint32_t)(wgs < 0xFFFFFFFFull ? wgs : 0xFFFFFFFFull) : 0u;
    }
    a.values = values;
    a.out_values = out_values;
    a.out_idx = out_indices;
    a.states = reinterpret_cast<tk::RowState*>(ws + p.off_states);
    a.call = reinterpret_cast<tk::CallState*>(ws + p.off_call);
    a.flagged = reinterpret_cast<uint32_t*>(ws + p.off_flag);
    a.ghist = reinterpret_cast<uint32_t*>(ws + p.off_ghist);
    a.skeys = reinterpret_cast<uint32_t*>(ws + p.off_skeys);
    a.shist = reinterpret_cast<uint32_t*>(ws + p.off_shist);
    a.cbuf = reinterpret_cast<uint64_t*>(ws + p.off_cbuf);
    a.aux = reinterpret_cast<uint64_t*>(ws + p.off_aux);
    a.lkc = reinterpret_cast<uint32_t*>(ws + p.off_lkc);
    a.lks = reinterpret_cast<uint64_t*>(ws + p.off_lks);
    a.rctr = reinterpret_cast<tk::RowCtr*>(ws + p.off_rctr);
    const uint64_t ctr = g_calls.fetch_add(1, std::memory_order_relaxed);
    a.seed = (params && params->use_seed) ? params->seed
                                          : (0x243F6A8885A308D3ull ^ (ctr * 0x9E3779B97F4A7C15ull));
    a.stream = static_cast<hipStream_t>(stream);
    if (allow_marks && g_prof.load(std::memory_order_relaxed)) a.mark = mark_stage;
    hipError_t e = tk::launch_pipeline(a);
    return e == hipSuccess ? TOPK_OK : TOPK_EHIP;
  } catch (const std::bad_alloc&) {
    return TOPK_EINVAL;
  } catch (...) {
    return TOPK_EINVAL;
  }
}

}  // namespace

extern "C" {

int topk_ex(const void* values, int64_t n, int64_t rows, int64_t k, int dtype, void* out_values,
            int64_t* out_indices, void* workspace, size_t workspace_bytes, void* stream,
            const topk_params* params) {
  return topk_run(values, n, rows, k, dtype, out_values, out_indices, workspace, workspace_bytes,
                  stream, params, true);
}

int topk_noalloc(const void* values, int64_t n, int64_t rows, int64_t k, int dtype,
                 void* out_values, int64_t* out_indices, void* stream,
                 const topk_params* params) {
  static_assert(tk::NOALLOC_SCRATCH_BYTES == (size_t)TOPK_NOALLOC_SCRATCH_BYTES,
                "the header states the scratch size");
  if (!values || !out_values || !out_indices) return TOPK_EINVAL;
  try {
    tk::Plan p;
    const int rc = plan_of(n, rows, k, dtype, params, &p, true);
    if (rc) return rc;
    if (p.total > tk::NOALLOC_SCRATCH_BYTES) return TOPK_ETOOBIG;
  } catch (...) {
    return TOPK_EINVAL;
  }
  void* ws = nullptr;
  if (tk::noalloc_scratch(&ws) != hipSuccess) return TOPK_EHIP;
  return topk_run(values, n, rows, k, dtype, out_values, out_indices, ws,
                  tk::NOALLOC_SCRATCH_BYTES, stream, params, false);
}

int topk(const void* values, int64_t n, int64_t rows, int64_t k, int dtype, void* out_values,
         int64_t* out_indices, void* workspace, size_t workspace_bytes, void* stream) {
  return topk_ex(values, n, rows, k, dtype, out_values, out_indices, workspace, workspace_bytes,
                 stream, nullptr);
}

int topk_read_stats(const void* workspace, int64_t rows, topk_row_stats* out, void* stream) {
  if (!workspace || !out || rows < 1 || rows > 65535) return TOPK_EINVAL;
  try {
    std::vector<tk::RowState> st((size_t)rows);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the row records follow the 256-byte header; the call record follows them
    const size_t off_states = sizeof(tk::WsHeader);
    if (hipMemcpyAsync(st.data(), static_cast<const char*>(workspace) + off_states,
                       sizeof(tk::RowState) * (size_t)rows, hipMemcpyDeviceToHost, s) != hipSuccess)
      return TOPK_EHIP;
    tk::CallState cs;
    const size_t off_call = (off_states + (size_t)rows * sizeof(tk::RowState) + 255) & ~(size_t)255;
    if (hipMemcpyAsync(&cs, static_cast<const char*>(workspace) + off_call, sizeof(cs),
                       hipMemcpyDeviceToHost, s) != hipSuccess)
      return TOPK_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TOPK_EHIP;
    for (int64_t r = 0; r < rows; ++r) {
      out[r].flags = cs.error;
      out[r].tau_key = st[(size_t)r].tau_key;
      out[r].r_sampled = st[(size_t)r].r_sampled;
      out[r].path = st[(size_t)r].path;
      out[r].passes = st[(size_t)r].passes;
      out[r].ties = st[(size_t)r].ties;
      out[r].tau_route = st[(size_t)r].tau_route;
    }
    return TOPK_OK;
  } catch (...) {
    return TOPK_EINVAL;
  }
}

int topk_filter_trace(uint64_t* buf, size_t words) {
  if (buf && reinterpret_cast<uintptr_t>(buf) % 8) return TOPK_EINVAL;
  g_trace_words.store(buf ? (uint64_t)words : 0);
  g_trace_buf.store(buf && words >= 2 ? buf : nullptr);
  return TOPK_OK;
}

int topk_profile_enable(int on) {
  g_prof.store(on ? 1 : 0);
  return TOPK_OK;
}

int topk_profile_read(topk_stage_times* out) {
  if (!out) return TOPK_EINVAL;
  std::memset(out, 0, sizeof(*out));
  std::lock_guard<std::mutex> g(g_prof_mu);
  int rc = TOPK_OK;
  for (const Bracket& br : g_done) {
    float ms = 0.f;
    if (hipEventSynchronize(br.b) != hipSuccess || hipEventElapsedTime(&ms, br.a, br.b) != hipSuccess)
      rc = TOPK_EHIP;
    out->ms[br.stage] += ms;
    out->count[br.stage] += 1;
    g_pool.push_back(br.a);
    g_pool.push_back(br.b);
  }
  g_done.clear();
  return rc;
}

int topk_scatter(const void* values, const int64_t* indices, int64_t rows, int64_t k, int64_t n,
                 int dtype, void* out_dense, uint8_t* out_mask, void* stream) {
  if (dtype != TOPK_I32 && dtype != TOPK_F32 && dtype != TOPK_BF16) return TOPK_EDTYPE;
  if (rows < 0 || k < 0 || n < 0 || k > n || (!out_dense && !out_mask)) return TOPK_EINVAL;
  if (rows * k > 0 && (!values || !indices)) return TOPK_EINVAL;
  const uintptr_t es = (dtype == TOPK_BF16) ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(values) % es || reinterpret_cast<uintptr_t>(out_dense) % es ||
      reinterpret_cast<uintptr_t>(indices) % 8)
    return TOPK_EINVAL;
  if ((uint64_t)rows * (uint64_t)k > 0xFFFFFFFFull * 256ull) return TOPK_EINVAL;
  const hipError_t e = tk::launch_scatter(values, indices, (uint64_t)rows, (uint64_t)k, (uint64_t)n,
                                          dtype,
                                          out_dense, out_mask, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TOPK_OK : TOPK_EHIP;
}

int topk_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream) {
  if (!data || !sink || bytes == 0) return TOPK_EINVAL;
  if (reinterpret_cast<uintptr_t>(data) % 16 || bytes % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return TOPK_EINVAL;
  const hipError_t e = tk::launch_stream_read(data, bytes, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TOPK_OK : TOPK_EHIP;
}

const char* topk_status_string(int status) {
  switch (status) {
    case TOPK_OK: return "ok";
    case TOPK_EINVAL: return "invalid argument";
    case TOPK_EDTYPE: return "unknown dtype";
    case TOPK_EWORKSPACE: return "workspace too small";
    case TOPK_EHIP: return "HIP error";
    case TOPK_ENOTIMPL: return "not implemented";
    case TOPK_ETOOBIG: return "call needs more scratch than topk_noalloc's built-in array";
    default: return "unknown status";
  }
}

}  // extern "C"
