/*
 * Plain CPU oracle for packed variable-length attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes (the plain definition, evaluated in IEEE fp64):
 *
 *   For every segment b with query rows [cu_q[b], cu_q[b+1]) and key rows
 *   [cu_k[b], cu_k[b+1]), every head h and every requested query row i of
 *   that segment:
 *       s_j   = scale * sum_d q[i,h,d] * k[j,h,d]        (j over the segment's keys)
 *       m     = max_j s_j                               (pass 1)
 *       l     = sum_j exp(s_j - m)                      (pass 2)
 *       o[d]  = sum_j exp(s_j - m) * v[j,h,d] / l
 *       lse   = m + ln(l)
 *   An empty key segment gives o = 0 and lse = -inf.
 *
 *   Causal variant (oracle_attn_varlen_fwd_causal): query row r of segment b
 *   (0-based within the segment, Lq = cu_q[b+1]-cu_q[b], Lk likewise) sees
 *   only the keys j (0-based within the segment) with j <= r + Lk - Lq, i.e.
 *   the mask is aligned to the bottom-right corner of the Lq x Lk score
 *   matrix, the flash-attention convention. The pages only call the
 *   interface with causal=False, so the alignment is a reading, not a fact
 *   they state. A row that sees no key gives o = 0 and lse = -inf.
 *
 * Sources: the softmax(Q K^T / sqrt(D)) V forward with its log-sum-exp that
 * the flash-attention varlen interface returns ("[FA4] cute varlen backward:
 * int32 overflow in _bwd_preprocess ..." page, "Real-world trigger" and the
 * repro script's forward call returning (out, lse)); packed segments given by
 * cumulative cu_seqlens for queries and keys ("[FA4][SM120] flash_attn_varlen_func
 * ... illegal memory access at >=4 varlen segments" page, "Bug 2 details",
 * captured call with cu_seqlens_q and max_seqlen_q/k); SDPA as the numerical
 * ground truth ("ffpa-attn PR #387" page, "Verification": numerics compared
 * against SDPA). Segments never interact: queries of segment b only see the
 * keys and values of segment b.
 *
 * The softmax is deliberately the two-pass (max, then sum) form and not an
 * online/streaming one. Inputs are bf16 bit patterns widened exactly to
 * double. Tensors are contiguous [tokens, H, D].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    const int32_t *cu_q, *cu_k;
    int32_t num_segments, num_heads, head_dim;
    double scale;
    const int64_t *rows; /* global query row per work item group */
    int64_t num_rows;
    double *out, *lse;
    int64_t item_begin, item_end; /* work items are (row index, head) pairs */
    int64_t max_keys;
    int32_t causal;
    int status;
} oracle_job;

/* Segment that owns global query row `row`, or -1. */
static int32_t segment_of_row(const int32_t *cu_q, int32_t num_segments, int64_t row) {
    int32_t lo = 0, hi = num_segments - 1;
    while (lo <= hi) {
        int32_t mid = lo + (hi - lo) / 2;
        if (row < (int64_t)cu_q[mid]) {
            hi = mid - 1;
        } else if (row >= (int64_t)cu_q[mid + 1]) {
            lo = mid + 1;
        } else {
            return mid;
        }
    }
    return -1;
}

static void one_row_one_head(const oracle_job *job, int64_t r, int32_t h, double *scores) {
    const int32_t H = job->num_heads, D = job->head_dim;
    const int64_t row = job->rows ? job->rows[r] : r;
    const int32_t b = segment_of_row(job->cu_q, job->num_segments, row);
    double *o = job->out + (r * H + h) * D;
    const int64_t k0 = job->cu_k[b], k1 = job->cu_k[b + 1];
    int64_t nk = k1 - k0;
    if (job->causal) {
        /* keys j <= (row - cu_q[b]) + Lk - Lq are visible */
        const int64_t lq = (int64_t)job->cu_q[b + 1] - job->cu_q[b];
        const int64_t visible = (row - job->cu_q[b]) + nk - lq + 1;
        nk = visible < 0 ? 0 : (visible < nk ? visible : nk);
    }
    if (nk == 0) {
        for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
        job->lse[r * H + h] = -INFINITY;
        return;
    }
    const uint16_t *qi = job->q + (row * H + h) * D;

    /* scores */
    for (int64_t j = 0; j < nk; ++j) {
        const uint16_t *kj = job->k + ((k0 + j) * H + h) * D;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += bf16_bits_to_double(qi[d]) * bf16_bits_to_double(kj[d]);
        scores[j] = job->scale * dot;
    }
    /* pass 1: maximum */
    double m = scores[0];
    for (int64_t j = 1; j < nk; ++j)
        if (scores[j] > m) m = scores[j];
    /* pass 2: weights, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const uint16_t *vj = job->v + ((k0 + j) * H + h) * D;
        for (int32_t d = 0; d < D; ++d) o[d] += scores[j] * bf16_bits_to_double(vj[d]);
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= l;
    job->lse[r * H + h] = m + log(l);
}

static void *run_job(void *arg) {
    oracle_job *job = (oracle_job *)arg;
    double *scores = (double *)malloc((size_t)(job->max_keys > 0 ? job->max_keys : 1) * sizeof(double));
    if (!scores) {
        job->status = -1;
        return NULL;
    }
    for (int64_t it = job->item_begin; it < job->item_end; ++it)
        one_row_one_head(job, it / job->num_heads, (int32_t)(it % job->num_heads), scores);
    free(scores);
    job->status = 0;
    return NULL;
}

static int run_all(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu_q,
                   const int32_t *cu_k, int32_t num_segments, int32_t num_heads, int32_t head_dim,
                   double scale, const int64_t *rows, int64_t num_rows, double *out, double *lse,
                   int32_t num_threads, int32_t causal) {
    if (!cu_q || !cu_k || num_segments < 0 || num_heads <= 0 || head_dim <= 0 || num_rows < 0)
        return -1;
    if (num_rows == 0) return 0;
    if (!q || !k || !v || !out || !lse || num_segments == 0) return -1;
    if (cu_q[0] != 0 || cu_k[0] != 0) return -1;
    int64_t max_keys = 0;
    for (int32_t b = 0; b < num_segments; ++b) {
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return -1;
        int64_t nk = (int64_t)cu_k[b + 1] - cu_k[b];
        if (nk > max_keys) max_keys = nk;
    }
    if (!rows && num_rows != cu_q[num_segments]) return -1;
    for (int64_t r = 0; rows && r < num_rows; ++r)
        if (segment_of_row(cu_q, num_segments, rows[r]) < 0) return -1;

    if (num_threads < 1) num_threads = 1;
    const int64_t items = num_rows * num_heads;
    if ((int64_t)num_threads > items) num_threads = (int32_t)items;
    oracle_job *jobs = (oracle_job *)calloc((size_t)num_threads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)num_threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    int rc = 0;
    int32_t started = 0;
    for (int32_t t = 0; t < num_threads; ++t) {
        oracle_job *j = &jobs[t];
        j->q = q; j->k = k; j->v = v; j->cu_q = cu_q; j->cu_k = cu_k;
        j->num_segments = num_segments; j->num_heads = num_heads; j->head_dim = head_dim;
        j->scale = scale; j->rows = rows; j->num_rows = num_rows; j->out = out; j->lse = lse;
        j->item_begin = items * t / num_threads;
        j->item_end = items * (t + 1) / num_threads;
        j->max_keys = max_keys;
        j->causal = causal;
        j->status = -1;
        if (t == 0) continue; /* the calling thread does slice 0 */
        if (pthread_create(&tids[t], NULL, run_job, j) != 0) {
            rc = -1;
            break;
        }
        started = t;
    }
    if (rc == 0) run_job(&jobs[0]);
    for (int32_t t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    for (int32_t t = 0; rc == 0 && t < num_threads; ++t)
        if (jobs[t].status != 0) rc = -1;
    free(jobs);
    free(tids);
    return rc;
}

/*
 * Evaluate attention for the query rows listed in `rows` (global token indices
 * into q), or for every query row when `rows` is NULL (then num_rows must be
 * cu_q[num_segments]).
 *   q: [Nq, H, D], k and v: [Nk, H, D] contiguous bf16 bit patterns.
 *   out: [num_rows, H, D] doubles; lse: [num_rows, H] doubles (natural log).
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int oracle_attn_varlen_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *cu_q, const int32_t *cu_k, int32_t num_segments,
                           int32_t num_heads, int32_t head_dim, double scale,
                           const int64_t *rows, int64_t num_rows, double *out, double *lse,
                           int32_t num_threads) {
    return run_all(q, k, v, cu_q, cu_k, num_segments, num_heads, head_dim, scale, rows, num_rows,
                   out, lse, num_threads, 0);
}

/* The same with the bottom-right aligned causal mask described above. */
int oracle_attn_varlen_fwd_causal(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  const int32_t *cu_q, const int32_t *cu_k, int32_t num_segments,
                                  int32_t num_heads, int32_t head_dim, double scale,
                                  const int64_t *rows, int64_t num_rows, double *out,
                                  double *lse, int32_t num_threads) {
    return run_all(q, k, v, cu_q, cu_k, num_segments, num_heads, head_dim, scale, rows, num_rows,
                   out, lse, num_threads, 1);
}
