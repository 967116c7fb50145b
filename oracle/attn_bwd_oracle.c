/*
 * Plain CPU oracle for the backward of packed variable-length attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes: the exact gradient of the forward in attn_oracle.c with
 * respect to q, k and v, for a given upstream gradient dout = dL/dO, in IEEE
 * fp64. For every segment b, head h and query row i of the segment, with the
 * keys j the row sees (all of the segment's, or with the causal mask the
 * bottom-right aligned prefix, as in the forward):
 *     s_j   = scale * q_i . k_j
 *     p_j   = exp(s_j - m) / l      (m = max_j s_j, l = sum_j exp(s_j - m); two passes)
 *     dp_j  = dout_i . v_j          (dL/dp_j, since o_i = sum_j p_j v_j)
 *     D_i   = sum_j p_j dp_j        (equals dout_i . o_i)
 *     ds_j  = p_j (dp_j - D_i)      (softmax Jacobian: dL/ds_j)
 *     dq_i  = scale * sum_j ds_j k_j
 *     dk_j += scale * ds_j q_i
 *     dv_j += p_j dout_i
 * A row that sees no key has o = 0 independent of q, k and v: it adds
 * nothing anywhere and its dq is 0.
 *
 * Sources: the backward of flash_attn_varlen_func (the "[FA4] cute varlen
 * backward: int32 overflow in _bwd_preprocess ..." page, "Summary" and the
 * repro's autograd call producing dQ/dK/dV from out and dout); the page names
 * the preprocessing kernel but gives no formula, so D_i above is the plain
 * reading of a per-row reduction over dout and out. The chain rule through
 * the softmax is mathematics, not taken from the page.
 *
 * Inputs are bf16 bit patterns widened exactly to double; tensors are
 * contiguous [tokens, H, D].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    const int32_t *cu_q, *cu_k;
    int32_t num_segments, num_heads, head_dim, causal;
    double scale;
    /* full mode: dq [Nq,H,D], dk/dv [Nk,H,D]; rows mode: dq [num_rows,H,D] only */
    const int64_t *rows;
    int64_t num_rows;
    double *dq, *dk, *dv;
    int64_t item_begin, item_end, max_keys;
    int status;
} bwd_job;

static int32_t owner_segment(const int32_t *cu_q, int32_t nseg, int64_t row) {
    int32_t lo = 0, hi = nseg - 1;
    while (lo <= hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        if (row < (int64_t)cu_q[mid])
            hi = mid - 1;
        else if (row >= (int64_t)cu_q[mid + 1])
            lo = mid + 1;
        else
            return mid;
    }
    return -1;
}

/* Keys of segment b that query row `row` (global) sees. */
static int64_t seen_keys(const bwd_job *job, int32_t b, int64_t row) {
    const int64_t lk = (int64_t)job->cu_k[b + 1] - job->cu_k[b];
    if (!job->causal) return lk;
    const int64_t lq = (int64_t)job->cu_q[b + 1] - job->cu_q[b];
    const int64_t n = (row - job->cu_q[b]) + lk - lq + 1;
    return n < 0 ? 0 : (n < lk ? n : lk);
}

/*
 * One query row and head: writes dq_i to dq_row and, when dk/dv are given,
 * adds the row's contributions to the key rows of its segment.
 * p and dp are scratch of at least max_keys doubles.
 */
static void bwd_row(const bwd_job *job, int64_t row, int32_t h, double *dq_row, double *dk,
                    double *dv, double *p, double *dp) {
    const int32_t H = job->num_heads, D = job->head_dim;
    const int32_t b = owner_segment(job->cu_q, job->num_segments, row);
    const int64_t k0 = job->cu_k[b];
    const int64_t nk = seen_keys(job, b, row);
    for (int32_t d = 0; d < D; ++d) dq_row[d] = 0.0;
    if (nk == 0) return;
    const uint16_t *qi = job->q + (row * H + h) * D;
    const uint16_t *gi = job->dout + (row * H + h) * D;

    for (int64_t j = 0; j < nk; ++j) {
        const uint16_t *kj = job->k + ((k0 + j) * H + h) * D;
        const uint16_t *vj = job->v + ((k0 + j) * H + h) * D;
        double s = 0.0, g = 0.0;
        for (int32_t d = 0; d < D; ++d) {
            s += widen(qi[d]) * widen(kj[d]);
            g += widen(gi[d]) * widen(vj[d]);
        }
        p[j] = job->scale * s;
        dp[j] = g;
    }
    double m = p[0];
    for (int64_t j = 1; j < nk; ++j)
        if (p[j] > m) m = p[j];
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    double Di = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        p[j] /= l;
        Di += p[j] * dp[j];
    }
    for (int64_t j = 0; j < nk; ++j) {
        const double ds = p[j] * (dp[j] - Di);
        const uint16_t *kj = job->k + ((k0 + j) * H + h) * D;
        for (int32_t d = 0; d < D; ++d) dq_row[d] += ds * widen(kj[d]);
        if (dk) {
            double *dkj = dk + ((k0 + j) * H + h) * D;
            double *dvj = dv + ((k0 + j) * H + h) * D;
            for (int32_t d = 0; d < D; ++d) {
                dkj[d] += job->scale * ds * widen(qi[d]);
                dvj[d] += p[j] * widen(gi[d]);
            }
        }
    }
    for (int32_t d = 0; d < D; ++d) dq_row[d] *= job->scale;
}

static void *bwd_run(void *arg) {
    bwd_job *job = (bwd_job *)arg;
    const size_t n = (size_t)(job->max_keys > 0 ? job->max_keys : 1);
    double *p = (double *)malloc(n * sizeof(double));
    double *dp = (double *)malloc(n * sizeof(double));
    if (!p || !dp) {
        free(p);
        free(dp);
        job->status = -1;
        return NULL;
    }
    const int32_t H = job->num_heads, D = job->head_dim;
    for (int64_t it = job->item_begin; it < job->item_end; ++it) {
        if (job->rows) {
            /* rows mode: item = (sampled row, head) */
            const int64_t r = it / H;
            const int32_t h = (int32_t)(it % H);
            bwd_row(job, job->rows[r], h, job->dq + (r * H + h) * D, NULL, NULL, p, dp);
        } else {
            /* full mode: item = (segment, head); its key rows belong to this job alone */
            const int32_t b = (int32_t)(it / H);
            const int32_t h = (int32_t)(it % H);
            for (int64_t row = job->cu_q[b]; row < job->cu_q[b + 1]; ++row)
                bwd_row(job, row, h, job->dq + (row * H + h) * D, job->dk, job->dv, p, dp);
        }
    }
    free(p);
    free(dp);
    job->status = 0;
    return NULL;
}

static int bwd_all(bwd_job proto, int32_t num_threads) {
    if (!proto.cu_q || !proto.cu_k || proto.num_segments <= 0 || proto.num_heads <= 0 ||
        proto.head_dim <= 0 || !proto.q || !proto.k || !proto.v || !proto.dout || !proto.dq)
        return -1;
    if (proto.cu_q[0] != 0 || proto.cu_k[0] != 0) return -1;
    int64_t max_keys = 0;
    for (int32_t b = 0; b < proto.num_segments; ++b) {
        if (proto.cu_q[b + 1] < proto.cu_q[b] || proto.cu_k[b + 1] < proto.cu_k[b]) return -1;
        const int64_t nk = (int64_t)proto.cu_k[b + 1] - proto.cu_k[b];
        if (nk > max_keys) max_keys = nk;
    }
    proto.max_keys = max_keys;
    int64_t items;
    if (proto.rows) {
        if (proto.num_rows < 0) return -1;
        for (int64_t r = 0; r < proto.num_rows; ++r)
            if (owner_segment(proto.cu_q, proto.num_segments, proto.rows[r]) < 0) return -1;
        items = proto.num_rows * proto.num_heads;
    } else {
        if (!proto.dk || !proto.dv) return -1;
        const int64_t H = proto.num_heads, D = proto.head_dim;
        memset(proto.dk, 0, (size_t)proto.cu_k[proto.num_segments] * H * D * sizeof(double));
        memset(proto.dv, 0, (size_t)proto.cu_k[proto.num_segments] * H * D * sizeof(double));
        items = (int64_t)proto.num_segments * proto.num_heads;
    }
    if (items == 0) return 0;
    if (num_threads < 1) num_threads = 1;
    if ((int64_t)num_threads > items) num_threads = (int32_t)items;
    bwd_job *jobs = (bwd_job *)calloc((size_t)num_threads, sizeof(bwd_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)num_threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    int rc = 0;
    int32_t started = 0;
    for (int32_t t = 0; t < num_threads; ++t) {
        jobs[t] = proto;
        jobs[t].item_begin = items * t / num_threads;
        jobs[t].item_end = items * (t + 1) / num_threads;
        jobs[t].status = -1;
        if (t == 0) continue;
        if (pthread_create(&tids[t], NULL, bwd_run, &jobs[t]) != 0) {
            rc = -1;
            break;
        }
        started = t;
    }
    if (rc == 0) bwd_run(&jobs[0]);
    for (int32_t t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    for (int32_t t = 0; rc == 0 && t < num_threads; ++t)
        if (jobs[t].status != 0) rc = -1;
    free(jobs);
    free(tids);
    return rc;
}

/*
 * Full gradients. q, dout: [Nq,H,D]; k, v: [Nk,H,D] contiguous bf16 bits.
 * dq: [cu_q[B],H,D], dk and dv: [cu_k[B],H,D] doubles (overwritten).
 * causal: 0 or 1 (mask as in the forward oracle). Returns 0, or -1 on bad arguments.
 */
int oracle_attn_varlen_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const uint16_t *dout, const int32_t *cu_q, const int32_t *cu_k,
                           int32_t num_segments, int32_t num_heads, int32_t head_dim,
                           double scale, int32_t causal, double *dq, double *dk, double *dv,
                           int32_t num_threads) {
    bwd_job j;
    memset(&j, 0, sizeof j);
    j.q = q; j.k = k; j.v = v; j.dout = dout; j.cu_q = cu_q; j.cu_k = cu_k;
    j.num_segments = num_segments; j.num_heads = num_heads; j.head_dim = head_dim;
    j.causal = causal != 0; j.scale = scale; j.dq = dq; j.dk = dk; j.dv = dv;
    return bwd_all(j, num_threads);
}

/*
 * dq only, for the global query rows listed in `rows` (each row is
 * independent of the others): dq is [num_rows,H,D] doubles.
 */
int oracle_attn_varlen_bwd_dq_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const uint16_t *dout, const int32_t *cu_q,
                                   const int32_t *cu_k, int32_t num_segments,
                                   int32_t num_heads, int32_t head_dim, double scale,
                                   int32_t causal, const int64_t *rows, int64_t num_rows,
                                   double *dq, int32_t num_threads) {
    if (!rows) return -1;
    bwd_job j;
    memset(&j, 0, sizeof j);
    j.q = q; j.k = k; j.v = v; j.dout = dout; j.cu_q = cu_q; j.cu_k = cu_k;
    j.num_segments = num_segments; j.num_heads = num_heads; j.head_dim = head_dim;
    j.causal = causal != 0; j.scale = scale; j.rows = rows; j.num_rows = num_rows; j.dq = dq;
    return bwd_all(j, num_threads);
}
