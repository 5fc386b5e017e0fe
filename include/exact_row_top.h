/*
 * exact_row_top.h -- C ABI of the MI355X (gfx950) exact per-row top-K library.
 *
 * The operation is the exact top-K selection a sparse-attention (DSA) indexer
 * runs over one fp32 score row per query, as stated on the TensorRT-LLM pages:
 *
 *  - "Self-sampling GVR V2 prefill indexer top-K" (PR 18702), section
 *    "Kernel": per row r, the top-K of logits[r, ks:ke] with ks = row_starts[r]
 *    and ke = row_ends[r], written in the row's LOCAL frame (column - ks) with a
 *    trailing -1 pad, and the identity 0..nv-1 when nv = ke - ks <= K.
 *  - "Block-skip fast path for self-sampling GVR top-K decode" (PR 18122),
 *    first commit message ("Contract"): fp32 scores, K in {512, 1024, 2048},
 *    exact top-K in which indices may interchange only inside the K-th value's
 *    tie class; the short-row commit (identity then -1); the varlen commit
 *    (per-row valid lengths read on the device, no host reads).
 *
 * How it is computed (Guess-Verify-Refine, PR 20998 "GVR K=2048 reg_clus with
 * block64 sampling and parallel rescue", sections "Why the GLM row overflows"
 * and "What changes"): sample K scores as K/64 blocks of 64 spread over the
 * row, bracket the K-th value with the sample's min/max, histogram the row
 * against that bracket, find the bin where the count from the top crosses K,
 * keep the bins above it, compact the crossing bin's members as candidates and
 * refine them exactly; an invalid bracket or an oversized crossing bin takes an
 * exact radix-select rescue over the whole row inside the same launch.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    never frees or retains them.  Calls are stream-ordered on `stream`
 *    (NULL = the null stream): the host never waits, never reads device data
 *    and, when `workspace` is given, never allocates.
 *  - logits: fp32 [num_rows][row_stride], unit inner stride, base 16-byte
 *    aligned, row_stride a multiple of 4 floats (the float4 row-stride gate of
 *    PR 18702's format check).  Every row's full stride must be readable: the
 *    kernel loads whole aligned float4 groups, and masks lanes outside the
 *    window by position, so values outside [ks, ke) (poison) never reach the
 *    selection.
 *  - indices: int32 [num_rows][k], 4-byte aligned.  Long rows (nv > k) get k
 *    distinct positions in [0, nv) in unspecified order; short rows get
 *    0..nv-1 then -1.
 *  - NaN inside a window is outside the contract (PR 18122, the commit that
 *    documents run_varlen's inherited NaN-ordering limitation): the kernels
 *    stay memory-safe on such a row (every read and write stays inside the
 *    row's stride, its k output slots and the workspace), but the k indices
 *    written for it are unspecified: they need not be distinct, nor inside
 *    the window.  +-inf are ordinary values; -0 and +0 are equal.
 *  - workspace: optional caller-owned device buffer of at least
 *    topk_workspace_bytes(...) bytes, 16-byte aligned (TOPK_ELAYOUT
 *    otherwise: the split tier moves its counts as 16-byte words), zeroed
 *    ONCE by topk_workspace_init before
 *    its first use; every call returns it to that resting state (histograms,
 *    cursors and counters back to zero), so a captured graph can replay
 *    without a memset.  The
 *    split tier's row barriers need the workgroups of a launch to be resident
 *    together; the plan bounds each launch by the device's resident capacity,
 *    so kernels that pin the GPU's compute units for their whole lifetime must
 *    not run beside these calls; a row barrier that waits too long gives up,
 *    the call's results are then undefined, and topk_status reports it.
 *    Calls that run concurrently (different streams) must not share one
 *    workspace (PR 18122, "varlen engine and seam" commit: a caller
 *    workspace so that concurrent streams do not share the split tier's
 *    publish slab).  NULL selects a per-device slab (PR 18122, first commit:
 *    per-device workspace slab) the library allocates on first need, zeroes
 *    before the call returns, keeps until process exit, and grows only when a
 *    larger plan needs it (allocation is not capture-safe).  There is one slab
 *    per GPU: calls with a NULL workspace must all go to one stream, or be
 *    ordered across streams by the caller.
 *  - Return value: TOPK_OK or one of the TOPK_E* codes below; nothing else
 *    crosses the ABI (no exceptions).  Argument errors are detected on the
 *    host before anything is launched.
 */
#ifndef EXACT_ROW_TOP_H_
#define EXACT_ROW_TOP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TOPK_OK = 0,
  TOPK_EINVAL = 1,     /* null pointer with num_rows > 0, num_rows < 0, k not in
                          {512,1024,2048}, row_stride < 1 or >= 2^30, bad option
                          value, a row longer than the largest launch plan
                          (64 workgroups x 512 threads x 9 float4 groups:
                          1,179,648 scores from the 16-byte boundary below
                          the window's start) */
  TOPK_ELAYOUT = 2,    /* logits not 16-byte aligned, row_stride % 4 != 0,
                          indices / extents not 4-byte aligned, a caller
                          workspace the plan uses not 16-byte aligned */
  TOPK_EWORKSPACE = 3, /* caller workspace smaller than topk_workspace_bytes
                          (topk_decode_noalloc: a plan larger than its fixed
                          scratch) */
  TOPK_EDEVICE = 4,    /* current device is not gfx950, or no device */
  TOPK_ELAUNCH = 5,    /* a HIP launch or allocation failed */
};

/* Decode form (PR 18122 varlen contract with next_n = 1, compress ratio 1):
 * row r selects from logits[r, 0:nv) with nv = clamp(n_valid[r], 0,
 * row_stride).  n_valid: device int32[num_rows]. */
int topk_decode(const float* logits, int64_t row_stride, const int32_t* n_valid,
                int32_t num_rows, int32_t k, int32_t* indices, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* Prefill form (PR 18702 "Kernel"): row r selects from logits[r, ks:ke) with
 * ks = clamp(row_starts[r], 0, row_stride), ke = clamp(row_ends[r], ks,
 * row_stride); indices are ks-relative.  row_starts / row_ends: device
 * int32[num_rows].  max_row_len: advisory host-side bound on ke - ks (0 =
 * none, < 0 rejected).  Launch shapes are always sized for row_stride, so any
 * window inside the stride is handled whatever the hint says. */
int topk_prefill(const float* logits, int64_t row_stride, const int32_t* row_starts,
                 const int32_t* row_ends, int32_t num_rows, int32_t k, int32_t* indices,
                 int64_t max_row_len, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Decode form that allocates nothing, for callers that cannot call hipMalloc
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same selection as topk_decode with a NULL workspace, but
 * the multi-workgroup tier keeps its state in a fixed per-GPU scratch array
 * of the library (24 MiB, held from library load until process exit) instead
 * of a caller workspace or the library's slab.  Plans whose workspace would
 * exceed it give TOPK_EWORKSPACE (no decode plan on a 256-compute-unit GPU
 * does).  The first call on a GPU clears the array with a kernel on
 * `stream`; every call returns it to zero.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, without
 * ordering between them) race and their results are undefined.  A row
 * barrier that gives up is counted by topk_status, whose reset also re-zeroes
 * the array. */
int topk_decode_noalloc(const float* logits, int64_t row_stride, const int32_t* n_valid,
                        int32_t num_rows, int32_t k, int32_t* indices, hipStream_t stream);

/* ---- Output options -------------------------------------------------------
 * Same selection as topk_decode / topk_prefill, with:
 *  values: optional device float[num_rows][k] (NULL = none), 4-byte aligned.
 *      values[r][i] is the score at indices[r][i] (logits[r, ks + idx]); short
 *      rows (nv <= k) keep their identity indices and pad values with
 *      -FLT_MAX (PR 18122, values-output commit).
 *  flags: TOPK_SORTED orders each long row's indices (and values) by value
 *      descending, then index ascending; TOPK_DETERMINISTIC resolves the K-th
 *      value's tie class by smallest index, so the selected set is the same on
 *      every call (PR 20998 "What changes" and "Walkthrough": smallest-index
 *      deterministic ties, optional output sorting).  With both flags a long
 *      row's output is its canonical top-k: positions ordered by value
 *      descending, equal values by position ascending.  Short rows are always
 *      identity + -1.  Unknown flag bits give TOPK_EINVAL.
 * Values and sorting run as a second kernel on the same stream. */
#define TOPK_SORTED 1u
#define TOPK_DETERMINISTIC 2u

int topk_decode_v(const float* logits, int64_t row_stride, const int32_t* n_valid,
                  int32_t num_rows, int32_t k, int32_t* indices, float* values, uint32_t flags,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

int topk_prefill_v(const float* logits, int64_t row_stride, const int32_t* row_starts,
                   const int32_t* row_ends, int32_t num_rows, int32_t k, int32_t* indices,
                   float* values, uint32_t flags, int64_t max_row_len, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* Varlen / MTP decode form (PR 18122, run_varlen commit: the production
 * decode contract): kv_lens is a device int32 array with one TOTAL cache length
 * per request, in uncompressed token space; row r belongs to request
 * r / next_n and selects from logits[r, 0:n) with
 *     n = (kv_lens[r / next_n] - next_n + r % next_n + 1) / compress_ratio
 * (integer division), no window when kv_lens[r / next_n] < next_n, and n
 * clamped to row_stride.  kv_lens needs ceil(num_rows / next_n) entries.
 * next_n >= 1 (MTP rows per request) and compress_ratio >= 1 (1 and 4 in the
 * pages' models), else TOPK_EINVAL.  values / flags as in topk_decode_v. */
int topk_decode_varlen(const float* logits, int64_t row_stride, const int32_t* kv_lens,
                       int32_t num_rows, int32_t next_n, int32_t compress_ratio, int32_t k,
                       int32_t* indices, float* values, uint32_t flags, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* ---- Hint-guided guess ----------------------------------------------------
 * Decode forms that also take the previous decode step's top-K positions as
 * hints (PR 18122 run_varlen commit: request-level raw pre_idx shared by a
 * request's next_n rows; "hint-robustness" commit and PR 20998 "What
 * changes": hints only steer the guess, exactness never depends on them).
 *  pre_idx: device int32, one row of at least k entries per request (per row
 *      in the plain decode form), pre_idx_stride (>= k, else TOPK_EINVAL)
 *      entries apart, 4-byte aligned.  Entries are raw positions in the
 *      row's window; any value is allowed: -1, positions at or past the
 *      window end and duplicates are ignored or harmless.  The guess reads
 *      the first min(k, workgroup size) entries of a hint row (256 to 1024;
 *      keep the hints of a row in no particular order, e.g. as a selection
 *      returns them).  NULL = no hints (the calls then equal topk_decode_v /
 *      topk_decode_varlen).
 * The result is the same exact selection as without hints, whatever the
 * hints hold.  Hints steer the multi-workgroup tier (the bracket's top and
 * floor); hints whose scores give no usable bracket (all invalid, all one
 * position) change nothing.  One-workgroup rows do not read them: their
 * retry takes the row's own maximum. */
int topk_decode_hinted(const float* logits, int64_t row_stride, const int32_t* n_valid,
                       const int32_t* pre_idx, int64_t pre_idx_stride, int32_t num_rows, int32_t k,
                       int32_t* indices, float* values, uint32_t flags, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

int topk_decode_varlen_hinted(const float* logits, int64_t row_stride, const int32_t* kv_lens,
                              const int32_t* pre_idx, int64_t pre_idx_stride, int32_t num_rows,
                              int32_t next_n, int32_t compress_ratio, int32_t k, int32_t* indices,
                              float* values, uint32_t flags, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ---- Block-skip pass --------------------------------------------------------
 * Decode form with per-32-score block maxima (PR 18122 "Description" and its
 * block-skip commit): the pass reads bmax and visits only the score blocks
 * whose maximum can reach the sampled threshold, then selects exactly as the
 * other forms do (same result, same output options).
 *  bmax: device float [num_rows][bmax_stride], bmax_stride >= ceil(row_stride
 *      / 32) (else TOPK_EINVAL), 4-byte aligned.  bmax[r][i] must be at least
 *      every score of logits[r, 32i : 32i + 32) inside the row's window (an
 *      upper bound suffices: NaN or +inf make a block always visited); with a
 *      smaller value the result is unspecified.  topk_block_max writes the
 *      exact maxima (the indexer GEMM's epilogue would in production).
 *  Gate (shape only): num_rows * row_stride * 4 >= 128 MiB and row_stride >=
 *  72 * k; other calls take the ordinary decode path, bmax unused.  The pass
 *  uses no workspace; hints are not used by it.
 *  Without bmax, decode calls of at least 128 rows whose row_stride exceeds
 *  what one resident workgroup holds (36864) and spans at least 4 * k blocks
 *  of 32 (up to 8192) take the pass in its streaming form, which makes the
 *  maxima itself (topk_options.blockskip = -1 keeps the resident tiers). */
int topk_decode_blockskip(const float* logits, int64_t row_stride, const int32_t* n_valid,
                          const float* bmax, int64_t bmax_stride, int32_t num_rows, int32_t k,
                          int32_t* indices, float* values, uint32_t flags, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* bmax[r][i] = max over logits[r, 32i : min(32i + 32, row_stride)) (NaN
 * ignored unless the whole block is NaN), for i < ceil(row_stride / 32). */
int topk_block_max(const float* logits, int64_t row_stride, int32_t num_rows, float* bmax,
                   int64_t bmax_stride, hipStream_t stream);

/* ---- Caller workspace and status ----------------------------------------
 * The pages' runner takes an optional caller workspace (PR 18122: run_ws
 * with a caller workspace, first commit; run_varlen(workspace=...) in the
 * "varlen engine and seam" commit, so that concurrent streams do not share
 * one publish slab).  These calls size, prepare and audit one. */

/* Bytes of workspace a call with num_rows rows of stride `max_row_len` needs
 * (pass the row_stride of the call; 0 when the plan uses one workgroup per
 * row and needs none).  The value does not depend on the device.  Returns 0
 * for invalid arguments as well.  Host only: no device access. */
size_t topk_workspace_bytes(int32_t num_rows, int64_t max_row_len, int32_t k);

/* Zero a workspace once before its first use: a stream-ordered memset of
 * workspace_bytes bytes of the caller's device buffer (the library keeps no
 * reference to it).  workspace NULL with workspace_bytes 0 is a no-op;
 * NULL with a size gives TOPK_EINVAL; a failed memset TOPK_ELAUNCH.  Not for
 * use inside a captured graph (it records a memset node); a zeroed workspace
 * stays zeroed between calls, so a graph needs none. */
int topk_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Stream-ordered audit of the split tier's bounded waits on the current
 * device.  Writes to *timeouts (device int32, 4-byte aligned) the number of
 * row-barrier waits that gave up since the previous topk_status on this
 * device, then resets that count.  A non-zero count means some call since
 * then returned undefined indices (its workgroups were not all resident
 * together: another kernel held compute units).  When the count is non-zero
 * the same launch also re-zeroes the library-owned slab; any caller
 * workspace used since then must be re-zeroed with topk_workspace_init
 * before its next use.  Two kernels on `stream`, no allocation, no host
 * sync; timeouts NULL gives TOPK_EINVAL. */
int topk_status(int32_t* timeouts, hipStream_t stream);

/* Static text for a status code (the pages' calls raise contract errors
 * loudly instead of falling back: PR 18122, the run_varlen production commit
 * and its fp32-contract commit).  Never NULL; unknown codes give
 * "unknown status". */
const char* topk_strerror(int status);

/* ---- Test and diagnostic surface ------------------------------------------
 * Same operations with knobs for tests.  `opts` may be NULL (= defaults).
 *  force_wgs_per_row: 0 = automatic plan; 1 = one workgroup per row; G > 1 =
 *      G workgroups per row (G <= 64), subject to the plan still fitting.
 *  force_rescue: nonzero = treat every long row's bracket as invalid, so the
 *      exact radix rescue runs on every long row.
 *  row_stats: optional device int32[num_rows][TOPK_STATS_WORDS]; per row:
 *      [0] path (0 short, 1 bracket + refine, 2 rescue: invalid bracket,
 *          3 rescue: crossing bin over the candidate cap (after the
 *          recounts below, where they apply), 5 fast path after a recount:
 *          a split row whose counts above its floor fell short of k counted
 *          again with no floor; a one-workgroup row whose crossing bin was
 *          the crowded top bin counted that bin again up to the row's
 *          maximum),
 *      [1] m (crossing-bin population, -1 if not computed),
 *      [2] above (count in bins above the crossing bin, -1 if none),
 *      [3] crossing bin index (-1 if none),
 *      [4] bit pattern of the bracket's low end (the sample minimum, or the
 *          lowest hint score when hints steered it), [5] of its high end,
 *      [6] workgroups per row, [7] candidate cap,
 *      [8] split rows: the floor bin the row's histogram counts from (-1 for
 *          one-workgroup rows and rows without a valid bracket); block-skip
 *          rows: the score blocks the last walk visited.
 *  Block-skip rows report path 1 (survivors only), 5 (counts short of k: every
 *  block recounted without a floor), 3 (crossing bin over the member cap) or 2
 *  (invalid bracket or forced rescue: radix select over the whole row).
 */
#define TOPK_STATS_WORDS 9

typedef struct topk_options {
  int32_t force_wgs_per_row;
  int32_t force_rescue;
  int32_t* row_stats;
  float* values;   /* as in topk_decode_v */
  uint32_t flags;  /* as in topk_decode_v */
  const int32_t* pre_idx; /* as in topk_decode_hinted (decode forms only,
                             else TOPK_EINVAL) */
  int64_t pre_idx_stride;
  const float* bmax;      /* as in topk_decode_blockskip (decode forms only) */
  int64_t bmax_stride;
  int32_t blockskip;      /* with bmax: 0 = the gate decides, 1 = always the
                             block-skip pass, -1 = never; 2 = the pass with
                             maxima it makes itself in a first streaming pass
                             (decode forms, rows of at most 8192 blocks of
                             32; bmax unused) */
  int32_t barrier_spins;  /* polls a split-tier row-barrier wait makes before
                             it gives up: 0 = the default (2^24, about a
                             second), n > 0 = n; < 0 gives TOPK_EINVAL.
                             Small values make waits give up on purpose
                             (undefined results, counted by topk_status):
                             for tests of that path only. */
} topk_options;

int topk_decode_ex(const float* logits, int64_t row_stride, const int32_t* n_valid,
                   int32_t num_rows, int32_t k, int32_t* indices, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, const topk_options* opts);

int topk_prefill_ex(const float* logits, int64_t row_stride, const int32_t* row_starts,
                    const int32_t* row_ends, int32_t num_rows, int32_t k, int32_t* indices,
                    int64_t max_row_len, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, const topk_options* opts);

int topk_decode_varlen_ex(const float* logits, int64_t row_stride, const int32_t* kv_lens,
                          int32_t num_rows, int32_t next_n, int32_t compress_ratio, int32_t k,
                          int32_t* indices, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, const topk_options* opts);

/* Host-only planning and validation, callable without a GPU.  Fills
 * out[0..6] = {workgroups per row, float4 groups per thread, rows per launch,
 * launches, workspace bytes, candidate cap, workgroup size} for the shapes
 * given (the same
 * plan topk_decode / topk_prefill would use; `force_wgs_per_row` as in
 * topk_options; `cu_count` and `wgs_per_cu` stand in for the device's resident
 * capacity).  Returns a status code. */
int topk_plan_query(int32_t num_rows, int64_t row_stride, int64_t max_row_len, int32_t k,
                    int32_t force_wgs_per_row, int32_t cu_count, int32_t wgs_per_cu,
                    int64_t* out);

/* Facts about the current device the planner uses (out holds 37 values):
 * out[0] = compute units; for k = {512, 1024, 2048}[ki] and the qi-th split
 * variant, out[1 + 3*ki + qi] = resident split-tier workgroups per compute
 * unit the planner uses, out[10 + ..] = the runtime occupancy figure,
 * out[19 + ..] = VGPRs per thread, out[28 + ..] = static LDS bytes.
 * Returns a status. */
int topk_device_query(int64_t* out);

/* Workspace layout (host-only): out[0] = error header bytes, out[1] = bytes
 * of each slot's fixed block (header, rescue digit counts, row histogram:
 * every word rests at zero between calls), out[2] = slots, out[3] = byte
 * offset of the per-slot data blocks; a plan with G workgroups per row has
 * data blocks of G * out[4] + out[5] bytes (out[4] = one workgroup's slice of
 * suffix counts, one 16-bit count per value bin; out[5] = the crossing-bin
 * member list).  Returns a status. */
int topk_workspace_layout(int64_t* out);

/* Measurement aid (not a selection): reads exactly the scores the selection
 * of the same call would read -- the windows of rows longer than k, as
 * aligned float4 groups -- in the launch shape the selection's plan uses
 * (one workgroup per row, or G per row with the same part split), and does
 * nothing else with them.  Its time is the floor the row reads alone set
 * under the selection's time.  mode 0: decode (extents = n_valid); mode 1:
 * prefill (extents = row_starts, extents2 = row_ends).  sink: device
 * uint32[1], written only on a data-dependent condition that keeps the loads.
 * Block-skip and streaming forms are not modelled.  Status as for
 * topk_decode. */
int topk_read_floor(int32_t mode, const float* logits, int64_t row_stride, const int32_t* extents,
                    const int32_t* extents2, int32_t num_rows, int32_t k, uint32_t* sink,
                    hipStream_t stream);

/* Host-side argument validation exactly as the entry points run it (no device
 * access).  mode: 0 decode (extents = n_valid, extents2 unused), 1 prefill. */
int topk_validate(int32_t mode, const void* logits, int64_t row_stride, const void* extents,
                  const void* extents2, int32_t num_rows, int32_t k, const void* indices,
                  const void* workspace, size_t workspace_bytes, int64_t max_row_len);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ROW_TOP_H_ */
