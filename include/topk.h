/*
 * topk.h - C ABI of the MI355X exact top-k selection library (libtopk_mi355x).
 *
 * What it computes: for each of `rows` contiguous rows of `n` elements, the k
 * largest entries together with their indices (Prof-K paper, section 3
 * "Problem Setup"; a batch applies the selection to each row).  The output is
 * in rank order: value descending, and on equal values the lower index first
 * (GPU.js Learn "Rank by Counting": an element is outranked by every larger
 * value and by every equal value at a lower index).  Values are compared as
 * follows (readings where the pages are silent): -0.0 equals +0.0; every NaN
 * ranks above +inf; NaNs tie with each other and are ordered by index.
 *
 * How: Prof-K one-pass filtering (section 3 "The Prof-K Algorithm" and
 * Algorithm 1): a device-side sample gives a threshold tau, one streaming
 * pass keeps every element >= tau in a bounded candidate buffer, and an exact
 * radix select plus sort of that buffer yields the answer.  If fewer than k
 * candidates survive or the buffer overflows, an exact radix select over the
 * full row runs instead, so the result is always the exact top-k.
 *
 * Conventions shared by every entry point
 *   - Device pointers are plain device addresses (memory from hipMalloc or a
 *     framework allocator); the caller owns all memory, the library allocates
 *     no device memory.
 *   - `values`: [rows, n] contiguous, element-aligned (4 bytes for int32 and
 *     float32, 2 bytes for bf16); 1 <= n < 2^32, rows >= 1, 1 <= k <= n.
 *   - `out_values`: [rows, k] of the input dtype; each output is the exact bit
 *     pattern of the selected input element.  `out_indices`: [rows, k] int64,
 *     row-local indices.
 *   - `workspace`: device memory of at least topk_workspace_size() bytes,
 *     256-byte aligned, owned by the caller.  It needs no initialisation and
 *     may hold anything between calls (another use of the same memory, a
 *     fresh allocation): every call writes each region before it reads it,
 *     resetting its per-call counters in its first kernel.  The one region
 *     kept from call to call is a sample histogram that a call leaves zero;
 *     the next call uses it only if the header's stamp names that call's
 *     layout, and otherwise rebuilds it (a little slower, same result).  One
 *     workspace must not be used by two calls that may run at the same time.
 *   - `stream`: a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; no host synchronisation happens
 *     inside topk/topk_ex.
 *   - Errors: argument problems return a negative status before anything is
 *     enqueued; a HIP launch failure returns TOPK_EHIP.  No exception crosses
 *     the ABI.
 *   - Exact route and co-residency.  The exact selection of the rows that
 *     fail the sampled check (or of every row, on the exact route) runs in one
 *     launch of one workgroup per compute unit whose phases wait for one
 *     another at grid barriers; that assumes all of its workgroups are
 *     resident at once.  When they are not (other work holding compute units
 *     for more than about 0.2 s, for instance two calls on different streams
 *     that both take the exact route at the same moment), every wait gives up
 *     after a bounded number of polls, the workgroups leave the shared phases,
 *     and the last one to finish selects each of those rows again on its own,
 *     exactly.  The answer is then still the exact top-k, the call takes far
 *     longer, and topk_read_stats reports it (flags bit 0).  For full speed,
 *     give calls that may run concurrently their own compute units or run
 *     them one after the other.
 */
#ifndef TOPK_MI355X_H
#define TOPK_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TOPK_I32 = 0, TOPK_F32 = 1, TOPK_BF16 = 2 } topk_dtype;

typedef enum {
  TOPK_OK = 0,
  TOPK_EINVAL = -1,     /* bad shape, k, pointer or alignment */
  TOPK_EDTYPE = -2,     /* unknown dtype */
  TOPK_EWORKSPACE = -3, /* workspace too small */
  TOPK_EHIP = -4,       /* a HIP call failed */
  TOPK_ENOTIMPL = -5,
  TOPK_ETOOBIG = -6     /* topk_noalloc: the call needs more than its scratch array */
} topk_status;

/* Parameter policy for (S, t, M).
 *  TOPK_POLICY_EXACT_TAIL: S from Algorithm 1; t and M the least values
 *    meeting the two conditions of Theorem 3 (recall failure R < k and
 *    overflow R > M each at most eps/2), evaluated with the exact
 *    hypergeometric law that Lemma 1 gives for the threshold rank.
 *  TOPK_POLICY_ALG1: Algorithm 1 verbatim (normal approximation of Lemma 2,
 *    t = 1 when alpha*S < -ln(eps/2)).
 *  TOPK_POLICY_TUNED (default): t and M as in EXACT_TAIL; S minimises the
 *    overhead of Eq. 13, tau_A*S + tau_B*M(S)*log2(k), with the exact-tail
 *    M(S) and tau_B/tau_A = tuned_ratio (k <= 4096, candidates refined in
 *    one workgroup), tuned_ratio_batched (k <= 4096 in calls of at least
 *    tuned_batch_rows rows: their samples are gathered together and cost
 *    bandwidth, while the rows refine side by side) or tuned_ratio_large
 *    (k > 4096, the multi-workgroup bucket sort), over the sample sizes
 *    tuned_s_min * 2^(j/4) (j = 0, 1, ...) up to min(s_max, n/8).  Sets S
 *    the way section 4 ("Optimal Sample Size") suggests, with the cost ratio
 *    measured on this engine instead of the default 1. */
typedef enum {
  TOPK_POLICY_EXACT_TAIL = 0,
  TOPK_POLICY_ALG1 = 1,
  TOPK_POLICY_TUNED = 2
} topk_policy;

/* Route.  AUTO: the sampled filter when n >= 8*S and the buffer M is below
 * n/2, except for rows of at most 2^18 elements where one workgroup per row
 * (exact, no sample) is estimated cheaper: about 8 us + 0.84 ns per element
 * per round of rows (a row per compute unit) against about 22 us + 0.025 us
 * per row + the input at 7 TB/s for the sampled route (MI355X timings).
 * Otherwise the exact radix select.  FILTER / EXACT force one route (FILTER
 * still falls back to the exact select when the sample fails). */
typedef enum { TOPK_PATH_AUTO = 0, TOPK_PATH_FILTER = 1, TOPK_PATH_EXACT = 2 } topk_path;

typedef struct {
  double eps;         /* failure budget, Algorithm 1 input (default 1e-3); EXACT_TAIL
                         and TUNED spend it per call: each of `rows` rows gets eps/rows */
  int64_t s_min;      /* sample size bounds (default 32768 and 131072) */
  int64_t s_max;
  double cost_ratio;  /* tau_B / tau_A of Eq. 13 in Algorithm 1 (default 1) */
  int32_t policy;     /* topk_policy */
  int32_t force_path; /* topk_path */
  uint64_t seed;      /* sampler seed when use_seed != 0 */
  int32_t use_seed;   /* 0: a fresh seed per call (a process-wide counter) */
  int32_t reserved;
  int64_t S;          /* > 0: override the sample size */
  int64_t t;          /* > 0: override the threshold rank */
  int64_t M;          /* > 0: override the buffer capacity */
  double tuned_ratio; /* TUNED policy, k <= 4096: tau_B / tau_A of this engine (default 0.13) */
  int64_t tuned_s_min;/* TUNED policy: least sample size considered (default 1024) */
  double tuned_ratio_large; /* TUNED policy, k > 4096: tau_B / tau_A (default 0.01) */
  double recall;      /* recall target rho in (0, 1] (default 1: exact).  Prof-K's
                         relaxed-recall trade (abstract; section 1): below 1 the
                         parameters are chosen for k_eff = ceil(rho * k) instead of
                         k, and a row where at least k_eff but fewer than k
                         elements reach tau (and they fit the buffer) keeps them
                         instead of taking the exact route.  Every one of them is a
                         true top-k element; they fill the first slots of the row
                         in rank order, and the remaining slots get index -1 and
                         the dtype's lowest value (-inf, or INT32_MIN).  Rows with
                         k or more survivors are exact as before. */
  uint32_t force_tau_key; /* with use_force_tau != 0: the threshold of every row, as
                         an order-preserving key (int32: bits ^ 0x80000000; float:
                         negatives all bits flipped, positives the sign bit set,
                         -0 as +0, every NaN 0xFFFFFFFF; bf16 the same on 16 bits).
                         The sampler is skipped and the sampled route runs with this
                         tau (Prof-K section 3, stages 3-4: filter, detection and the
                         fallback); the result is still the exact top-k.  Meant for
                         driving detection from the host, e.g. the largest key
                         forces R < k (section 4, "Failure Modes and Budget
                         Allocation").  Not allowed with force_path = EXACT. */
  int32_t use_force_tau;
  uint32_t test_flags;  /* test aid, 0 in normal use: TOPK_TEST_BARRIER_GIVEUP makes
                         every grid-barrier wait of the exact route give up at once,
                         as when workgroups are not co-resident.  Other bits: EINVAL. */
  int32_t tuned_batch_rows;   /* TUNED policy: least row count priced with
                         tuned_ratio_batched (default 32) */
  double tuned_ratio_batched; /* TUNED policy, k <= 4096 and rows >= tuned_batch_rows:
                         tau_B / tau_A (default 0.03) */
} topk_params;

enum { TOPK_TEST_BARRIER_GIVEUP = 1 };

/* Resolved plan of one call shape (host arithmetic only; no GPU needed). */
typedef struct {
  int32_t path;       /* 0 sampled filter, 1 exact multi-workgroup, 2 exact one workgroup per row */
  int32_t small_k;    /* 1: k winners sorted in one workgroup; 0: multi-workgroup sort */
  int64_t S, t, M;    /* sample size, threshold rank, buffer capacity (sampled route) */
  int64_t cap;        /* candidate buffer capacity per row */
  int32_t index_bits; /* B: bits of the index field of the composite */
  int32_t key_bits;   /* 32 (int32, float32) or 16 (bf16) */
  double p_recall;    /* P(R < k_eff) per row for distinct values (Lemma 1), sampled
                         route; k_eff = k unless params.recall < 1 */
  double p_overflow;  /* P(R > M) per row for distinct values (Lemma 1), sampled route */
  size_t workspace_bytes;
  int64_t k_eff;      /* the selection size the parameters were chosen for: k, or
                         ceil(params.recall * k) below recall 1 */
} topk_plan_info;

/* Per-row record of the last call on a workspace (topk_read_stats). */
typedef struct {
  uint32_t tau_key;   /* sampled threshold as an order-preserving key */
  uint32_t r_sampled; /* survivors of the sampled filter pass (R); on an
                         overflow the pass may stop early, and this is then
                         only some count above the buffer capacity */
  uint32_t path;      /* 0 sampled accepted, 1 sampled then exact fallback, 2 exact only,
                         3 sampled with fewer than k survivors kept (recall < 1) */
  uint32_t passes;    /* histogram passes of the exact select */
  uint32_t flags;     /* of the whole call: bit 0 = an exact-route grid-barrier wait
                         gave up (workgroups not co-resident; the rows of the exact
                         route were then selected again by one workgroup: the
                         result is exact, the call was slow); bit 1 = internal
                         limit of the large-k sort exceeded (never expected) */
  uint32_t ties;      /* of r_sampled, the survivors equal to tau; they join the
                         candidates only when fewer than k lie strictly above */
  uint32_t tau_route; /* diagnostic: how tau was selected.  Low 3 bits: 0 none (exact
                         route), 1 per-workgroup top-t lists in the filter's prologue,
                         2 top-t lists in the threshold kernel, 3 every sample key in
                         registers, 4 every sample key streamed, 5 given by the caller
                         (use_force_tau), 6 top-t lists radix-selected in the filter's
                         prologue, 7 sorted lists of 32 (t > 8) merged in the filter's
                         prologue.  Bit 3: the sample bin holding rank t had more
                         keys than LDS holds (streamed radix select); bit 4: that bin was
                         radix-selected in LDS. */
} topk_row_stats;

/* Fill *p with the defaults above.  Returns TOPK_OK, or TOPK_EINVAL for NULL. */
int topk_default_params(topk_params* p);

/* Plan of a call shape under `params` (NULL = defaults): Algorithm 1 and the
 * chosen policy, the route, the buffer capacity and the workspace size.
 * Host arithmetic only.  Errors: TOPK_EINVAL, TOPK_EDTYPE. */
int topk_plan(int64_t n, int64_t rows, int64_t k, int dtype, const topk_params* params,
              topk_plan_info* out);

/* Workspace bytes one call of this shape needs (params NULL = defaults). */
int topk_workspace_size(int64_t n, int64_t rows, int64_t k, int dtype, const topk_params* params,
                        size_t* bytes);

/* Zero-fill `bytes` of workspace on `stream` with a fill kernel (no memset
 * node, so it can sit inside a captured graph).  Optional: a workspace needs
 * no initialisation. */
int topk_workspace_init(void* workspace, size_t bytes, void* stream);

/* Exact top-k with default parameters.  See the conventions above. */
int topk(const void* values, int64_t n, int64_t rows, int64_t k, int dtype, void* out_values,
         int64_t* out_indices, void* workspace, size_t workspace_bytes, void* stream);

/* topk with explicit parameters (NULL = defaults).  The result is the exact
 * top-k whatever the parameters; they only move work between the sampled
 * route and the exact fallback. */
int topk_ex(const void* values, int64_t n, int64_t rows, int64_t k, int dtype, void* out_values,
            int64_t* out_indices, void* workspace, size_t workspace_bytes, void* stream,
            const topk_params* params);

/* topk_ex for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The workspace is a device array built into the
 * library, TOPK_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on
 * a GPU until the process ends; every call on a GPU uses that GPU's array.
 * Calls needing more (topk_workspace_size) return TOPK_ETOOBIG before
 * anything is enqueued.  No device allocation, free or memset: the array
 * needs no clearing, since every call writes what it reads (see the
 * workspace convention above).  Calls that may overlap on one GPU (other
 * streams, other threads) race on the array: run them one after another.
 * topk_read_stats is not available for these calls.  Same arguments,
 * results and errors as topk_ex otherwise. */
#define TOPK_NOALLOC_SCRATCH_BYTES (32u << 20)
int topk_noalloc(const void* values, int64_t n, int64_t rows, int64_t k, int dtype,
                 void* out_values, int64_t* out_indices, void* stream,
                 const topk_params* params);

/* Copy the per-row records of the last call on `workspace` into out[0..rows)
 * (host memory).  Synchronises `stream`.  Errors: TOPK_EINVAL, TOPK_EHIP. */
int topk_read_stats(const void* workspace, int64_t rows, topk_row_stats* out, void* stream);

/* Stage timing (measurement aid).  While enabled, each call records HIP
 * events on its stream around its stages; topk_profile_read waits for them
 * and returns the summed milliseconds and bracket counts per stage, then
 * forgets them.  Stage order: sample, tau, filter, refine, exact/fallback,
 * sort.  The events add a few microseconds per call. */
typedef struct {
  double ms[8];
  int64_t count[8];
} topk_stage_times;

int topk_profile_enable(int on);
int topk_profile_read(topk_stage_times* out);

/* Filter workgroup trace (measurement aid: how evenly the filter's
 * workgroups finish; Appendix D, "Efficient GPU Implementation", asks for a
 * pass at memory speed, which the slowest workgroup bounds).  While set,
 * every call's filter launch writes, for each of its workgroups l < words / 2
 * (l = row * workgroups per row + the workgroup's index in its row; workgroup
 * l runs on XCD l mod 8), the device's 100 MHz realtime counter at the
 * workgroup's start into buf[2 l] and at the end of its scan into
 * buf[2 l + 1].  buf: caller-owned device memory of `words` 64-bit words,
 * 8-byte aligned, written by later calls until replaced; NULL stops the
 * trace.  Process-wide; not synchronised with calls in flight.  Errors:
 * TOPK_EINVAL (misaligned buf). */
int topk_filter_trace(uint64_t* buf, size_t words);

/* BatchTopK consumer (Prof-K section 5, "Application: BatchTopK Sparse
 * Autoencoders": the batch-global top-k keeps the K largest of the flattened
 * B x d_dict activations).  Turns a selection into the sparse activation:
 * for every row r < rows and j < k, out_dense[r*n + indices[r*k + j]] =
 * values[r*k + j]; every other element of out_dense[0 .. rows*n) becomes 0.
 * out_mask, if not null, gets 1 at the same places and 0 elsewhere (one byte
 * per element).  values / indices are laid out as topk writes them (for the
 * flattened call rows = 1, n = B*d_dict, k = K); out_dense has the dtype of
 * values.  Either output may be null, not both.  An index outside [0, n) is
 * skipped (so the padded slots of a relaxed-recall selection, index -1,
 * write nothing).  All pointers are device memory; values and out_dense aligned to
 * the element size, indices to 8 bytes; the outputs must not overlap the
 * inputs.  Two kernels on `stream` (a zero fill, then one thread per
 * winner), asynchronous.  Errors: TOPK_EDTYPE, TOPK_EINVAL (sizes, k > n,
 * no output, alignment), TOPK_EHIP. */
int topk_scatter(const void* values, const int64_t* indices, int64_t rows, int64_t k, int64_t n,
                 int dtype, void* out_dense, uint8_t* out_mask, void* stream);

/* Read ceiling (measurement aid, not part of a selection).  Reads
 * data[0..bytes) once on `stream` with the filter's access pattern: one
 * 512-thread workgroup per compute unit, each streaming a contiguous slice
 * with four 16-byte nontemporal loads per lane in flight and the next four
 * issued before the current ones are used.  Nothing is written except,
 * with negligible probability, one word of sink[0..64) (caller-owned device
 * memory of 64 words).  Timing it gives the achievable read bandwidth of that
 * pattern, against which the filter's bandwidth is judged.  data must be
 * device memory, 16-byte aligned, bytes a non-zero multiple of 16; otherwise
 * TOPK_EINVAL.  Asynchronous; TOPK_EHIP if the launch fails. */
int topk_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream);

/* Short English text for a status code (static storage). */
const char* topk_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_MI355X_H */
