/*
 * oracle_topk.c -- plain, slow, exact per-row top-K on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes is the selection contract the pages state, written out as
 * its plain definition (no sampling, no histogram, no Guess-Verify-Refine):
 *
 *  - "Self-sampling GVR V2 prefill indexer top-K" (TensorRT-LLM PR 18702),
 *    section "Kernel": per row r the top-K of logits[r, ks:ke], reported in the
 *    row's LOCAL frame (column - ks) with a trailing -1 pad, and the identity
 *    0..nv-1 when nv = ke - ks <= K.
 *  - "Block-skip fast path ..." (PR 18122), first commit message: exact top-K
 *    in which indices may interchange only inside the K-th value's tie class,
 *    with signed zeros treated as equal; and the short-row commit: rows with
 *    no more than K valid entries emit identity indices padded with -1.
 *  - "GVR K=2048 reg_clus ..." (PR 20998), section "What changes": smallest-
 *    index tie choice is the deterministic form, which is the canonical output
 *    this oracle emits.
 *
 * Definition used, per row:
 *   1. Resolve the window with the boundary's clamps.  Decode: ks = 0,
 *      nv = clamp(n_valid[r], 0, row_stride).  Prefill: ks = clamp(row_starts
 *      [r], 0, row_stride), ke = clamp(row_ends[r], ks, row_stride).
 *   2. nv <= k: out = 0, 1, ..., nv-1, then -1 up to k entries.
 *   3. Otherwise sort the positions 0..nv-1 of the window by IEEE value,
 *      larger first, equal values (so -0 == +0) by smaller position first;
 *      out = the first k positions in that order.
 * A NaN inside a window is outside the contract (the varlen engine commit of
 * PR 18122 documents an inherited NaN-ordering limitation): such a row is
 * rejected -- its output is filled with INT32_MIN and it is counted in the
 * return value.  Infinities are ordinary values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    float v;
    int32_t pos;
} entry_t;

/* Larger value first; equal values (IEEE equality, so -0 == +0) by position. */
static int by_value_desc_then_pos(const void* pa, const void* pb) {
    const entry_t* a = (const entry_t*)pa;
    const entry_t* b = (const entry_t*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

/* Exact top-k of one window w[0..nv) (any k >= 1).  Returns 0, or 1 if the
 * window holds a NaN (row rejected).  `scratch` holds nv entries. */
int oracle_topk_window(const float* w, int64_t nv, int32_t k, int32_t* out,
                       void* scratch) {
    if (nv < 0) nv = 0;
    if (nv <= k) {
        for (int32_t i = 0; i < k; ++i) out[i] = (i < nv) ? i : -1;
        return 0;
    }
    entry_t* e = (entry_t*)scratch;
    for (int64_t i = 0; i < nv; ++i) {
        if (isnan(w[i])) {
            for (int32_t j = 0; j < k; ++j) out[j] = INT32_MIN;
            return 1;
        }
        e[i].v = w[i];
        e[i].pos = (int32_t)i;
    }
    qsort(e, (size_t)nv, sizeof(entry_t), by_value_desc_then_pos);
    for (int32_t j = 0; j < k; ++j) out[j] = e[j].pos;
    return 0;
}

static int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

typedef struct {
    const float* logits;
    int64_t row_stride;
    const int32_t* n_valid;    /* decode, or NULL */
    const int32_t* row_starts; /* prefill, or NULL */
    const int32_t* row_ends;
    int64_t num_rows;
    int32_t k;
    int32_t* out;
    int64_t next_row; /* shared work counter */
    pthread_mutex_t lock;
    int64_t rejected;
} job_t;

static void resolve(const job_t* j, int64_t r, int64_t* ks, int64_t* nv) {
    if (j->n_valid) {
        *ks = 0;
        *nv = clamp64(j->n_valid[r], 0, j->row_stride);
    } else {
        int64_t s = clamp64(j->row_starts[r], 0, j->row_stride);
        int64_t e = clamp64(j->row_ends[r], s, j->row_stride);
        *ks = s;
        *nv = e - s;
    }
}

static void* worker(void* arg) {
    job_t* j = (job_t*)arg;
    entry_t* scratch = (entry_t*)malloc(sizeof(entry_t) * (size_t)(j->row_stride + 1));
    int64_t rej = 0;
    for (;;) {
        pthread_mutex_lock(&j->lock);
        int64_t r = j->next_row++;
        pthread_mutex_unlock(&j->lock);
        if (r >= j->num_rows) break;
        int64_t ks, nv;
        resolve(j, r, &ks, &nv);
        rej += oracle_topk_window(j->logits + r * j->row_stride + ks, nv, j->k,
                                  j->out + r * (int64_t)j->k, scratch);
    }
    free(scratch);
    pthread_mutex_lock(&j->lock);
    j->rejected += rej;
    pthread_mutex_unlock(&j->lock);
    return NULL;
}

static int64_t run(job_t* j, int32_t nthreads) {
    if (nthreads <= 0) nthreads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > j->num_rows) nthreads = (int32_t)(j->num_rows > 0 ? j->num_rows : 1);
    j->next_row = 0;
    j->rejected = 0;
    pthread_mutex_init(&j->lock, NULL);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int32_t t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, worker, j);
    for (int32_t t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&j->lock);
    return j->rejected;
}

/* Decode form: logits [num_rows][row_stride] (host memory), n_valid[num_rows],
 * out [num_rows][k].  Rows are spread over `nthreads` threads (<= 0: all
 * online cores).  Returns the number of rejected (NaN) rows. */
int64_t oracle_topk_decode(const float* logits, int64_t row_stride,
                           const int32_t* n_valid, int64_t num_rows, int32_t k,
                           int32_t* out, int32_t nthreads) {
    job_t j;
    memset(&j, 0, sizeof(j));
    j.logits = logits;
    j.row_stride = row_stride;
    j.n_valid = n_valid;
    j.num_rows = num_rows;
    j.k = k;
    j.out = out;
    return run(&j, nthreads);
}

/* Prefill form: per-row windows [row_starts[r], row_ends[r]). */
int64_t oracle_topk_prefill(const float* logits, int64_t row_stride,
                            const int32_t* row_starts, const int32_t* row_ends,
                            int64_t num_rows, int32_t k, int32_t* out,
                            int32_t nthreads) {
    job_t j;
    memset(&j, 0, sizeof(j));
    j.logits = logits;
    j.row_stride = row_stride;
    j.row_starts = row_starts;
    j.row_ends = row_ends;
    j.num_rows = num_rows;
    j.k = k;
    j.out = out;
    return run(&j, nthreads);
}

int32_t oracle_online_cores(void) { return (int32_t)sysconf(_SC_NPROCESSORS_ONLN); }
