/*
 * CPU oracle for fused MaxSim scoring -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this library. The HIP library never links, calls or shares code
 * with it. It is a plain, slow, obviously correct evaluation of the
 * definitions, in double precision for floating-point inputs and in 64-bit
 * integers for int8 inputs, multithreaded only over independent outputs.
 *
 * Sources (page title, then the passage):
 *   [FM]  "Flash-MaxSim" (academ.us article 2605.29517):
 *         Eq. (1) MaxSim; Sec. 4.1.1 online max with -inf masking;
 *         Sec. 4.2.1 Eqs. (2)-(3) closed-form gradients;
 *         Sec. 4.2.2 inverse-grid CSR (bincount, cumsum, stable argsort);
 *         Sec. 4.3.1 INT8 x INT8 (per-tensor and per-token scales);
 *         Sec. 4.3.2 padding-free cu_seqlens.
 *   [TMS] "TileMaxSim: IO-Aware GPU MaxSim Scoring ..." (arXiv 2606.26439v1):
 *         Sec. 6.8 "End-to-End Retrieval Latency" (top-k after scoring).
 *   [LIK] "late-interaction-kernels design notes" (docs/design.md):
 *         "Problem" (masks), "Forward" pseudocode (strict '>' update,
 *         argmax starts at 0, finalise m <- finite(m) & q_active ? m : 0),
 *         "Backward" formulas with q_mask, "Varlen / packed path"
 *         (empty sequences contribute zero).
 *
 * Readings where the pages leave a step open:
 *   - ties go to the lowest doc-token index (strict '>' in ascending t);
 *   - a q-masked row still gets the real argmax; only its score term is 0;
 *   - a doc with no valid token contributes 0 and keeps argmax 0;
 *   - varlen argmax is [Nq, Nd, max_lq], doc-relative, rows past Lq_i are 0;
 *   - the CSR holds every source (i, j, s), masked ones included; masks enter
 *     the gradients only through w = g[i,j] * q_mask[i,s] * live(j), where
 *     live(j) says doc j has at least one valid token;
 *   - a CSR column index is the flat source index (i*Nd + j)*Lq + s.
 *
 * Every entry point returns 0 on success and a negative value when an input
 * breaks a stated precondition (argmax outside [0, Ld), non-monotone offsets).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* A minimal parallel-for: each worker takes a contiguous block of items.    */
/* ------------------------------------------------------------------------ */
typedef void (*item_fn)(void* ctx, int64_t item);

typedef struct {
    item_fn fn;
    void* ctx;
    int64_t lo, hi;
} span_t;

static void* run_span(void* p)
{
    span_t* s = (span_t*)p;
    for (int64_t k = s->lo; k < s->hi; ++k) s->fn(s->ctx, k);
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, item_fn fn, void* ctx)
{
    if (n <= 0) return;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > n) nthreads = (int)n;
    if (nthreads == 1) {
        for (int64_t k = 0; k < n; ++k) fn(ctx, k);
        return;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    span_t* sp = (span_t*)malloc(sizeof(span_t) * (size_t)nthreads);
    int started = 0;
    for (int w = 0; w < nthreads; ++w) {
        sp[w].fn = fn;
        sp[w].ctx = ctx;
        sp[w].lo = n * w / nthreads;
        sp[w].hi = n * (w + 1) / nthreads;
        if (pthread_create(&th[w], NULL, run_span, &sp[w]) != 0) break;
        ++started;
    }
    /* anything a failed thread creation left over runs here */
    for (int w = started; w < nthreads; ++w) run_span(&sp[w]);
    for (int w = 0; w < started; ++w) pthread_join(th[w], NULL);
    free(th);
    free(sp);
}

/* ------------------------------------------------------------------------ */
/* One (query, doc) pair of Eq. (1): sum over query rows s of the max over   */
/* valid doc rows t of <Q[s], D[t]>, following the Forward pseudocode.       */
/* ------------------------------------------------------------------------ */
static double pair_f64(const double* Qi, const double* Dj, int64_t Lq, int64_t Ld, int64_t d,
                       const uint8_t* qm, const uint8_t* dm, int32_t* arg)
{
    double acc = 0.0;
    for (int64_t s = 0; s < Lq; ++s) {
        const double* q = Qi + s * d;
        double best = -INFINITY;
        int64_t at = 0;
        for (int64_t t = 0; t < Ld; ++t) {
            if (dm && !dm[t]) continue; /* masked token is -inf: never selected */
            const double* x = Dj + t * d;
            double v = 0.0;
            for (int64_t k = 0; k < d; ++k) v += q[k] * x[k];
            if (v > best) { /* strict: the lowest index keeps a tie */
                best = v;
                at = t;
            }
        }
        if (arg) arg[s] = (int32_t)at;
        if (isfinite(best) && (!qm || qm[s])) acc += best;
    }
    return acc;
}

typedef struct {
    const double *Q, *D;
    int64_t Nq, Nd, Lq, Ld, d;
    const uint8_t *qm, *dm;
    double* scores;
    int32_t* argmax;
} dense_ctx;

static void dense_item(void* p, int64_t k)
{
    dense_ctx* c = (dense_ctx*)p;
    int64_t i = k / c->Nd, j = k % c->Nd;
    c->scores[k] = pair_f64(c->Q + i * c->Lq * c->d, c->D + j * c->Ld * c->d, c->Lq, c->Ld, c->d,
                            c->qm ? c->qm + i * c->Lq : NULL, c->dm ? c->dm + j * c->Ld : NULL,
                            c->argmax ? c->argmax + k * c->Lq : NULL);
}

/* Cross-product forward. Q [Nq,Lq,d], D [Nd,Ld,d]; masks [Nq,Lq], [Nd,Ld] of
 * 0/1 bytes or NULL; scores [Nq,Nd]; argmax [Nq,Nd,Lq] or NULL. */
int oracle_fwd_f64(const double* Q, const double* D, int64_t Nq, int64_t Nd, int64_t Lq,
                   int64_t Ld, int64_t d, const uint8_t* q_mask, const uint8_t* d_mask,
                   double* scores, int32_t* argmax, int nthreads)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return -1;
    dense_ctx c = {Q, D, Nq, Nd, Lq, Ld, d, q_mask, d_mask, scores, argmax};
    parallel_for(Nq * Nd, nthreads, dense_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Padding-free form: sequence b occupies rows [cu[b], cu[b+1]).             */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *Q, *D;
    const int32_t *cu_q, *cu_d;
    int64_t Nq, Nd, max_lq, d;
    double* scores;
    int32_t* argmax;
} varlen_ctx;

static void varlen_item(void* p, int64_t k)
{
    varlen_ctx* c = (varlen_ctx*)p;
    int64_t i = k / c->Nd, j = k % c->Nd;
    int64_t q0 = c->cu_q[i], lq = (int64_t)c->cu_q[i + 1] - q0;
    int64_t d0 = c->cu_d[j], ld = (int64_t)c->cu_d[j + 1] - d0;
    int32_t* arg = c->argmax ? c->argmax + k * c->max_lq : NULL;
    if (arg)
        for (int64_t s = 0; s < c->max_lq; ++s) arg[s] = 0;
    c->scores[k] = pair_f64(c->Q + q0 * c->d, c->D + d0 * c->d, lq, ld, c->d, NULL, NULL, arg);
}

int oracle_fwd_varlen_f64(const double* Q, const int32_t* cu_q, int64_t Nq, int64_t max_lq,
                          const double* D, const int32_t* cu_d, int64_t Nd, int64_t d,
                          double* scores, int32_t* argmax, int nthreads)
{
    if (Nq < 0 || Nd < 0 || d < 0 || max_lq < 0) return -1;
    for (int64_t i = 0; i < Nq; ++i) {
        int64_t l = (int64_t)cu_q[i + 1] - cu_q[i];
        if (l < 0 || l > max_lq) return -2;
    }
    for (int64_t j = 0; j < Nd; ++j)
        if (cu_d[j + 1] < cu_d[j]) return -2;
    varlen_ctx c = {Q, D, cu_q, cu_d, Nq, Nd, max_lq, d, scores, argmax};
    parallel_for(Nq * Nd, nthreads, varlen_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* INT8 x INT8 with one symmetric scale per tensor: exact integer max-sum,   */
/* then score = q_scale * d_scale * sum.                                     */
/* ------------------------------------------------------------------------ */
typedef struct {
    const int8_t *Q, *D;
    int64_t Nq, Nd, Lq, Ld, d;
    const uint8_t *qm, *dm;
    int64_t* score_i;
    double* score_f;
    double q_scale, d_scale;
    int32_t* argmax;
} i8_ctx;

static void i8_item(void* p, int64_t k)
{
    i8_ctx* c = (i8_ctx*)p;
    int64_t i = k / c->Nd, j = k % c->Nd;
    const int8_t* Qi = c->Q + i * c->Lq * c->d;
    const int8_t* Dj = c->D + j * c->Ld * c->d;
    const uint8_t* qm = c->qm ? c->qm + i * c->Lq : NULL;
    const uint8_t* dm = c->dm ? c->dm + j * c->Ld : NULL;
    int32_t* arg = c->argmax ? c->argmax + k * c->Lq : NULL;
    int64_t acc = 0;
    for (int64_t s = 0; s < c->Lq; ++s) {
        const int8_t* q = Qi + s * c->d;
        int found = 0;
        int64_t best = 0, at = 0;
        for (int64_t t = 0; t < c->Ld; ++t) {
            if (dm && !dm[t]) continue;
            const int8_t* x = Dj + t * c->d;
            int64_t v = 0;
            for (int64_t e = 0; e < c->d; ++e) v += (int64_t)q[e] * (int64_t)x[e];
            if (!found || v > best) {
                found = 1;
                best = v;
                at = t;
            }
        }
        if (arg) arg[s] = (int32_t)at;
        if (found && (!qm || qm[s])) acc += best;
    }
    c->score_i[k] = acc;
    if (c->score_f) c->score_f[k] = (double)acc * c->q_scale * c->d_scale;
}

int oracle_fwd_i8(const int8_t* Q, double q_scale, const int8_t* D, double d_scale, int64_t Nq,
                  int64_t Nd, int64_t Lq, int64_t Ld, int64_t d, const uint8_t* q_mask,
                  const uint8_t* d_mask, int64_t* score_i, double* score_f, int32_t* argmax,
                  int nthreads)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return -1;
    i8_ctx c = {Q, D, Nq, Nd, Lq, Ld, d, q_mask, d_mask, score_i, score_f, q_scale, d_scale, argmax};
    parallel_for(Nq * Nd, nthreads, i8_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward through the saved argmax: Eqs. (2)-(3) with the q_mask factor of */
/* the design notes, the CSR by counting sort (histogram, exclusive scan,    */
/* fill in ascending source order = stable argsort of destinations).         */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *Q, *D, *g;
    int64_t Nq, Nd, Lq, Ld, d;
    const uint8_t* qm;
    const uint8_t* live;
    const int32_t* argmax;
    const int32_t *row_ptr, *col_idx;
    double *dQ, *dD;
} bwd_ctx;

static double weight(const bwd_ctx* c, int64_t i, int64_t j, int64_t s)
{
    if (!c->live[j]) return 0.0;
    if (c->qm && !c->qm[i * c->Lq + s]) return 0.0;
    return c->g[i * c->Nd + j];
}

/* Eq. (2): dQ[i,s] = sum over j ascending of w * D[j, argmax[i,j,s]] */
static void dq_item(void* p, int64_t r)
{
    bwd_ctx* c = (bwd_ctx*)p;
    int64_t i = r / c->Lq, s = r % c->Lq;
    double* out = c->dQ + r * c->d;
    for (int64_t k = 0; k < c->d; ++k) out[k] = 0.0;
    for (int64_t j = 0; j < c->Nd; ++j) {
        double w = weight(c, i, j, s);
        if (w == 0.0) continue;
        int64_t t = c->argmax[(i * c->Nd + j) * c->Lq + s];
        const double* x = c->D + (j * c->Ld + t) * c->d;
        for (int64_t k = 0; k < c->d; ++k) out[k] += w * x[k];
    }
}

/* Eq. (3): dD[j,t] = sum over the sources listed in CSR row (j,t), in order */
static void dd_item(void* p, int64_t r)
{
    bwd_ctx* c = (bwd_ctx*)p;
    double* out = c->dD + r * c->d;
    for (int64_t k = 0; k < c->d; ++k) out[k] = 0.0;
    for (int64_t e = c->row_ptr[r]; e < c->row_ptr[r + 1]; ++e) {
        int64_t src = c->col_idx[e];
        int64_t s = src % c->Lq;
        int64_t ij = src / c->Lq;
        int64_t i = ij / c->Nd, j = ij % c->Nd;
        double w = weight(c, i, j, s);
        if (w == 0.0) continue;
        const double* q = c->Q + (i * c->Lq + s) * c->d;
        for (int64_t k = 0; k < c->d; ++k) out[k] += w * q[k];
    }
}

int oracle_bwd_f64(const double* Q, const double* D, int64_t Nq, int64_t Nd, int64_t Lq,
                   int64_t Ld, int64_t d, const uint8_t* q_mask, const uint8_t* d_mask,
                   const int32_t* argmax, const double* g, double* dQ, double* dD,
                   int32_t* row_ptr, int32_t* col_idx, int nthreads)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return -1;
    int64_t nsrc = Nq * Nd * Lq, nrows = Nd * Ld;
    if (nsrc > 0 && Ld == 0) return -2; /* no destination exists */
    for (int64_t e = 0; e < nsrc; ++e)
        if (argmax[e] < 0 || argmax[e] >= Ld) return -2;

    uint8_t* live = (uint8_t*)calloc((size_t)(Nd > 0 ? Nd : 1), 1);
    for (int64_t j = 0; j < Nd; ++j) {
        int any = 0;
        for (int64_t t = 0; t < Ld && !any; ++t) any = d_mask ? d_mask[j * Ld + t] != 0 : 1;
        live[j] = (uint8_t)any;
    }

    /* histogram of destinations (bincount) */
    int64_t* cnt = (int64_t*)calloc((size_t)(nrows + 1), sizeof(int64_t));
    for (int64_t src = 0; src < nsrc; ++src) {
        int64_t j = (src / Lq) % Nd;
        cnt[j * Ld + argmax[src]] += 1;
    }
    /* exclusive scan (cumsum shifted by one) */
    int64_t run = 0;
    for (int64_t r = 0; r < nrows; ++r) {
        row_ptr[r] = (int32_t)run;
        run += cnt[r];
    }
    row_ptr[nrows] = (int32_t)run;
    /* fill in ascending source order: the stable argsort of destinations */
    for (int64_t r = 0; r < nrows; ++r) cnt[r] = row_ptr[r];
    for (int64_t src = 0; src < nsrc; ++src) {
        int64_t j = (src / Lq) % Nd;
        int64_t r = j * Ld + argmax[src];
        col_idx[cnt[r]++] = (int32_t)src;
    }
    free(cnt);

    bwd_ctx c = {Q, D, g, Nq, Nd, Lq, Ld, d, q_mask, live, argmax, row_ptr, col_idx, dQ, dD};
    parallel_for(Nq * Lq, nthreads, dq_item, &c);
    parallel_for(nrows, nthreads, dd_item, &c);
    free(live);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* INT8 x INT8 with one symmetric scale per token ("Flash-MaxSim" Sec.       */
/* 4.3.1): the similarity of query row s and doc row t is the dot product of */
/* the dequantised rows, q_scale[s] * d_scale[t] * <Q8[s], D8[t]>, taken     */
/* through the same masked max and sum as Eq. (1).                           */
/* ------------------------------------------------------------------------ */
typedef struct {
    const int8_t *Q, *D;
    const double *qs, *ds;
    int64_t Nq, Nd, Lq, Ld, d;
    const uint8_t *qm, *dm;
    double* score;
    int32_t* argmax;
} i8tok_ctx;

static void i8tok_item(void* p, int64_t k)
{
    i8tok_ctx* c = (i8tok_ctx*)p;
    int64_t i = k / c->Nd, j = k % c->Nd;
    const int8_t* Qi = c->Q + i * c->Lq * c->d;
    const int8_t* Dj = c->D + j * c->Ld * c->d;
    const double* qs = c->qs + i * c->Lq;
    const double* ds = c->ds + j * c->Ld;
    const uint8_t* qm = c->qm ? c->qm + i * c->Lq : NULL;
    const uint8_t* dm = c->dm ? c->dm + j * c->Ld : NULL;
    int32_t* arg = c->argmax ? c->argmax + k * c->Lq : NULL;
    double acc = 0.0;
    for (int64_t s = 0; s < c->Lq; ++s) {
        const int8_t* q = Qi + s * c->d;
        double best = -INFINITY;
        int64_t at = 0;
        for (int64_t t = 0; t < c->Ld; ++t) {
            if (dm && !dm[t]) continue;
            const int8_t* x = Dj + t * c->d;
            int64_t dot = 0;
            for (int64_t e = 0; e < c->d; ++e) dot += (int64_t)q[e] * (int64_t)x[e];
            const double v = qs[s] * ds[t] * (double)dot;
            if (v > best) {
                best = v;
                at = t;
            }
        }
        if (arg) arg[s] = (int32_t)at;
        if (isfinite(best) && (!qm || qm[s])) acc += best;
    }
    c->score[k] = acc;
}

/* Q int8 [Nq,Lq,d] with q_scale [Nq,Lq]; D int8 [Nd,Ld,d] with d_scale
 * [Nd,Ld]; masks as in oracle_fwd_f64; score [Nq,Nd]; argmax or NULL. */
int oracle_fwd_i8_tok(const int8_t* Q, const double* q_scale, const int8_t* D,
                      const double* d_scale, int64_t Nq, int64_t Nd, int64_t Lq, int64_t Ld,
                      int64_t d, const uint8_t* q_mask, const uint8_t* d_mask, double* score,
                      int32_t* argmax, int nthreads)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0) return -1;
    i8tok_ctx c = {Q, D, q_scale, d_scale, Nq, Nd, Lq, Ld, d, q_mask, d_mask, score, argmax};
    parallel_for(Nq * Nd, nthreads, i8tok_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Top-k after scoring (the retrieval step that follows the scores in the    */
/* TileMaxSim paper, Sec. 6.8 "End-to-End Retrieval Latency"): for each      */
/* query the k largest scores in decreasing order; equal scores are taken in */
/* increasing doc order. A full sort under that total order, then the first  */
/* k entries.                                                                */
/* ------------------------------------------------------------------------ */
typedef struct {
    double v;
    int64_t j;
} scored_t;

static int scored_cmp(const void* a, const void* b)
{
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

typedef struct {
    const double* scores;
    int64_t Nd, K;
    int32_t* idx;
    double* val;
} topk_ctx;

static void topk_item(void* p, int64_t i)
{
    topk_ctx* c = (topk_ctx*)p;
    scored_t* a = (scored_t*)malloc(sizeof(scored_t) * (size_t)(c->Nd > 0 ? c->Nd : 1));
    for (int64_t j = 0; j < c->Nd; ++j) {
        a[j].v = c->scores[i * c->Nd + j];
        a[j].j = j;
    }
    qsort(a, (size_t)c->Nd, sizeof(scored_t), scored_cmp);
    for (int64_t r = 0; r < c->K; ++r) {
        c->idx[i * c->K + r] = (int32_t)a[r].j;
        c->val[i * c->K + r] = a[r].v;
    }
    free(a);
}

/* scores [Nq,Nd] (no NaN); idx [Nq,K] int32 and val [Nq,K]; 0 <= K <= Nd */
int oracle_topk(const double* scores, int64_t Nq, int64_t Nd, int64_t K, int32_t* idx,
                double* val, int nthreads)
{
    if (Nq < 0 || Nd < 0 || K < 0 || K > Nd) return -1;
    for (int64_t e = 0; e < Nq * Nd; ++e)
        if (isnan(scores[e])) return -2;
    topk_ctx c = {scores, Nd, K, idx, val};
    parallel_for(Nq, nthreads, topk_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Scores of listed (query, doc) pairs: Eq. (1) for pair p between query     */
/* pair_q[p] and doc pair_d[p] of the dense tensors (rescoring candidates).  */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *Q, *D;
    int64_t Nq, Nd, Lq, Ld, d;
    const uint8_t *qm, *dm;
    const int32_t *pq, *pd;
    double* scores;
    int32_t* argmax;
} pairs_ctx;

static void pairs_item(void* p, int64_t k)
{
    pairs_ctx* c = (pairs_ctx*)p;
    int64_t i = c->pq[k], j = c->pd[k];
    c->scores[k] = pair_f64(c->Q + i * c->Lq * c->d, c->D + j * c->Ld * c->d, c->Lq, c->Ld, c->d,
                            c->qm ? c->qm + i * c->Lq : NULL, c->dm ? c->dm + j * c->Ld : NULL,
                            c->argmax ? c->argmax + k * c->Lq : NULL);
}

int oracle_fwd_pairs_f64(const double* Q, const double* D, int64_t Nq, int64_t Nd, int64_t Lq,
                         int64_t Ld, int64_t d, const uint8_t* q_mask, const uint8_t* d_mask,
                         const int32_t* pair_q, const int32_t* pair_d, int64_t P, double* scores,
                         int32_t* argmax, int nthreads)
{
    if (Nq < 0 || Nd < 0 || Lq < 0 || Ld < 0 || d < 0 || P < 0) return -1;
    for (int64_t k = 0; k < P; ++k)
        if (pair_q[k] < 0 || pair_q[k] >= Nq || pair_d[k] < 0 || pair_d[k] >= Nd) return -2;
    pairs_ctx c = {Q, D, Nq, Nd, Lq, Ld, d, q_mask, d_mask, pair_q, pair_d, scores, argmax};
    parallel_for(P, nthreads, pairs_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Padding-free backward ([FM] Sec. 4.2.1 Eqs. (2)-(3) and Sec. 4.2.2 on the */
/* packed layout of Sec. 4.3.2; [LIK] "Varlen / packed path"). Query i is    */
/* packed rows [cu_q[i], cu_q[i+1]), doc j rows [cu_d[j], cu_d[j+1]). The    */
/* argmax is the forward's [Nq, Nd, max_lq] doc-relative map. Sources are    */
/* the real query rows (s < Lq_i) of every doc that has a token; an empty    */
/* doc has no destination row and contributes nothing. The CSR has one row   */
/* per packed doc token; a column index is the flat source index             */
/* (i*Nd + j)*max_lq + s, rows list their sources ascending.                 */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *Q, *D, *g;
    const int32_t *cu_q, *cu_d;
    int64_t Nq, Nd, max_lq, d;
    const int32_t* argmax;
    const int32_t *row_ptr, *col_idx;
    double *dQ, *dD;
} vbwd_ctx;

/* Eq. (2) for packed query row p: sum over live docs j ascending */
static void vdq_item(void* p_, int64_t i)
{
    vbwd_ctx* c = (vbwd_ctx*)p_;
    for (int64_t s = 0; s < (int64_t)c->cu_q[i + 1] - c->cu_q[i]; ++s) {
        double* out = c->dQ + ((int64_t)c->cu_q[i] + s) * c->d;
        for (int64_t k = 0; k < c->d; ++k) out[k] = 0.0;
        for (int64_t j = 0; j < c->Nd; ++j) {
            if (c->cu_d[j + 1] == c->cu_d[j]) continue; /* empty doc: no gradient */
            double w = c->g[i * c->Nd + j];
            int64_t t = c->argmax[(i * c->Nd + j) * c->max_lq + s];
            const double* x = c->D + ((int64_t)c->cu_d[j] + t) * c->d;
            for (int64_t k = 0; k < c->d; ++k) out[k] += w * x[k];
        }
    }
}

/* Eq. (3) for packed doc row r: the sources of CSR row r, in order */
static void vdd_item(void* p_, int64_t r)
{
    vbwd_ctx* c = (vbwd_ctx*)p_;
    double* out = c->dD + r * c->d;
    for (int64_t k = 0; k < c->d; ++k) out[k] = 0.0;
    for (int64_t e = c->row_ptr[r]; e < c->row_ptr[r + 1]; ++e) {
        int64_t src = c->col_idx[e];
        int64_t s = src % c->max_lq, ij = src / c->max_lq;
        int64_t i = ij / c->Nd, j = ij % c->Nd;
        double w = c->g[i * c->Nd + j];
        const double* q = c->Q + ((int64_t)c->cu_q[i] + s) * c->d;
        for (int64_t k = 0; k < c->d; ++k) out[k] += w * q[k];
    }
}

int oracle_bwd_varlen_f64(const double* Q, const int32_t* cu_q, int64_t Nq, int64_t max_lq,
                          const double* D, const int32_t* cu_d, int64_t Nd, int64_t d,
                          const int32_t* argmax, const double* g, double* dQ, double* dD,
                          int32_t* row_ptr, int32_t* col_idx, int nthreads)
{
    if (Nq < 0 || Nd < 0 || d < 0 || max_lq < 0) return -1;
    if ((Nq > 0 && cu_q[0] != 0) || (Nd > 0 && cu_d[0] != 0)) return -2;
    for (int64_t i = 0; i < Nq; ++i) {
        int64_t l = (int64_t)cu_q[i + 1] - cu_q[i];
        if (l < 0 || l > max_lq) return -2;
    }
    for (int64_t j = 0; j < Nd; ++j)
        if (cu_d[j + 1] < cu_d[j]) return -2;
    int64_t nrows = Nd > 0 ? cu_d[Nd] : 0;
    /* sources (i, j, s) in ascending flat index; destination row cu_d[j] + t */
    int64_t* cnt = (int64_t*)calloc((size_t)(nrows + 1), sizeof(int64_t));
    for (int64_t i = 0; i < Nq; ++i)
        for (int64_t j = 0; j < Nd; ++j) {
            int64_t ld = (int64_t)cu_d[j + 1] - cu_d[j];
            if (ld == 0) continue;
            for (int64_t s = 0; s < (int64_t)cu_q[i + 1] - cu_q[i]; ++s) {
                int64_t t = argmax[(i * Nd + j) * max_lq + s];
                if (t < 0 || t >= ld) {
                    free(cnt);
                    return -2;
                }
                cnt[cu_d[j] + t] += 1; /* histogram (bincount) */
            }
        }
    int64_t run = 0; /* exclusive scan */
    for (int64_t r = 0; r < nrows; ++r) {
        row_ptr[r] = (int32_t)run;
        run += cnt[r];
    }
    row_ptr[nrows] = (int32_t)run;
    for (int64_t r = 0; r < nrows; ++r) cnt[r] = row_ptr[r];
    for (int64_t i = 0; i < Nq; ++i) /* fill in ascending source order */
        for (int64_t j = 0; j < Nd; ++j) {
            if (cu_d[j + 1] == cu_d[j]) continue;
            for (int64_t s = 0; s < (int64_t)cu_q[i + 1] - cu_q[i]; ++s) {
                int64_t src = (i * Nd + j) * max_lq + s;
                col_idx[cnt[cu_d[j] + argmax[src]]++] = (int32_t)src;
            }
        }
    free(cnt);
    vbwd_ctx c = {Q, D, g, cu_q, cu_d, Nq, Nd, max_lq, d, argmax, row_ptr, col_idx, dQ, dD};
    parallel_for(Nq, nthreads, vdq_item, &c);
    parallel_for(nrows, nthreads, vdd_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Scores of listed (query, doc) pairs of packed batches ([LIK] "Varlen /    */
/* packed path", the pair-list scorer): pair p is Eq. (1) for query pair_q[p]*/
/* against doc pair_d[p]; argmax [P, max_lq] as the packed forward's.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *Q, *D;
    const int32_t *cu_q, *cu_d, *pq, *pd;
    int64_t max_lq, d;
    double* scores;
    int32_t* argmax;
} vpairs_ctx;

static void vpairs_item(void* p_, int64_t p)
{
    vpairs_ctx* c = (vpairs_ctx*)p_;
    int64_t i = c->pq[p], j = c->pd[p];
    int64_t q0 = c->cu_q[i], lq = (int64_t)c->cu_q[i + 1] - q0;
    int64_t d0 = c->cu_d[j], ld = (int64_t)c->cu_d[j + 1] - d0;
    int32_t* arg = c->argmax ? c->argmax + p * c->max_lq : NULL;
    if (arg)
        for (int64_t s = 0; s < c->max_lq; ++s) arg[s] = 0;
    c->scores[p] = pair_f64(c->Q + q0 * c->d, c->D + d0 * c->d, lq, ld, c->d, NULL, NULL, arg);
}

int oracle_fwd_pairs_varlen_f64(const double* Q, const int32_t* cu_q, int64_t Nq, int64_t max_lq,
                                const double* D, const int32_t* cu_d, int64_t Nd, int64_t d,
                                const int32_t* pair_q, const int32_t* pair_d, int64_t P,
                                double* scores, int32_t* argmax, int nthreads)
{
    if (Nq < 0 || Nd < 0 || d < 0 || max_lq < 0 || P < 0) return -1;
    for (int64_t i = 0; i < Nq; ++i) {
        int64_t l = (int64_t)cu_q[i + 1] - cu_q[i];
        if (l < 0 || l > max_lq) return -2;
    }
    for (int64_t j = 0; j < Nd; ++j)
        if (cu_d[j + 1] < cu_d[j]) return -2;
    for (int64_t p = 0; p < P; ++p)
        if (pair_q[p] < 0 || pair_q[p] >= Nq || pair_d[p] < 0 || pair_d[p] >= Nd) return -2;
    vpairs_ctx c = {Q, D, cu_q, cu_d, pair_q, pair_d, max_lq, d, scores, argmax};
    parallel_for(P, nthreads, vpairs_item, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Chamfer distance ([FM] Sec. 4.2.4): batch b holds point sets P[b] (N x 3) */
/* and Q[b] (M x 3). dist1[b,p] = min over q of ||p - q||^2 with idx1 the    */
/* lowest q attaining it; dist2/idx2 the same from Q to P; loss[b] =         */
/* (1/N) sum_p dist1 + (1/M) sum_q dist2. Squared distances are summed over  */
/* the 3 coordinates in fp64 from the exact fp32 inputs.                     */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *A, *Bp;
    int64_t na, nb;
    double* dist;
    int32_t* idx;
} cham_ctx;

/* item = (batch, source point): min over the batch's target points, ascending */
static void cham_item(void* p_, int64_t k)
{
    cham_ctx* c = (cham_ctx*)p_;
    int64_t b = k / c->na;
    const double* a = c->A + k * 3;
    const double* tgt = c->Bp + b * c->nb * 3;
    double best = INFINITY;
    int32_t arg = 0;
    for (int64_t t = 0; t < c->nb; ++t) {
        double dx = a[0] - tgt[t * 3], dy = a[1] - tgt[t * 3 + 1], dz = a[2] - tgt[t * 3 + 2];
        double v = dx * dx + dy * dy + dz * dz;
        if (v < best) { /* strict: the lowest index wins ties */
            best = v;
            arg = (int32_t)t;
        }
    }
    c->dist[k] = best;
    c->idx[k] = arg;
}

int oracle_chamfer_fwd(const double* P, const double* Q, int64_t B, int64_t N, int64_t M,
                       double* dist1, int32_t* idx1, double* dist2, int32_t* idx2, double* loss,
                       int nthreads)
{
    if (B < 0 || N < 0 || M < 0) return -1;
    if (B > 0 && (N == 0 || M == 0)) return -2; /* a min over an empty set */
    cham_ctx c1 = {P, Q, N, M, dist1, idx1};
    parallel_for(B * N, nthreads, cham_item, &c1);
    cham_ctx c2 = {Q, P, M, N, dist2, idx2};
    parallel_for(B * M, nthreads, cham_item, &c2);
    if (loss)
        for (int64_t b = 0; b < B; ++b) {
            double s1 = 0.0, s2 = 0.0;
            for (int64_t p = 0; p < N; ++p) s1 += dist1[b * N + p];
            for (int64_t q = 0; q < M; ++q) s2 += dist2[b * M + q];
            loss[b] = s1 / (double)N + s2 / (double)M;
        }
    return 0;
}

/* Inverse map of one direction by counting sort: sources k = b*ns + s with  */
/* destination row b*nr + idx[k]; rows list their sources ascending.         */
static void seg_csr(const int32_t* idx, int64_t B, int64_t ns, int64_t nr, int32_t* row_ptr,
                    int32_t* col_idx)
{
    int64_t nrows = B * nr, nsrc = B * ns;
    int64_t* cnt = (int64_t*)calloc((size_t)(nrows + 1), sizeof(int64_t));
    for (int64_t k = 0; k < nsrc; ++k) cnt[(k / ns) * nr + idx[k]] += 1;
    int64_t run = 0;
    for (int64_t r = 0; r < nrows; ++r) {
        row_ptr[r] = (int32_t)run;
        run += cnt[r];
    }
    row_ptr[nrows] = (int32_t)run;
    for (int64_t r = 0; r < nrows; ++r) cnt[r] = row_ptr[r];
    for (int64_t k = 0; k < nsrc; ++k) col_idx[cnt[(k / ns) * nr + idx[k]]++] = (int32_t)k;
    free(cnt);
}

/* Gradient of sum g1*dist1 + sum g2*dist2 at the saved argmins:            */
/*   dP[b,p] = 2 g1[b,p] (P[b,p] - Q[b,idx1]) + sum over CSR2 row (b,p) of  */
/*             2 g2[b,q] (P[b,p] - Q[b,q])                                  */
/*   dQ[b,q] = 2 g2[b,q] (Q[b,q] - P[b,idx2]) + sum over CSR1 row (b,q) of  */
/*             2 g1[b,p] (Q[b,q] - P[b,p])                                  */
int oracle_chamfer_bwd(const double* P, const double* Q, int64_t B, int64_t N, int64_t M,
                       const int32_t* idx1, const int32_t* idx2, const double* g1,
                       const double* g2, double* dP, double* dQ, int32_t* row_ptr1,
                       int32_t* col_idx1, int32_t* row_ptr2, int32_t* col_idx2)
{
    if (B < 0 || N < 0 || M < 0) return -1;
    if (B > 0 && (N == 0 || M == 0)) return -2;
    for (int64_t k = 0; k < B * N; ++k)
        if (idx1[k] < 0 || idx1[k] >= M) return -2;
    for (int64_t k = 0; k < B * M; ++k)
        if (idx2[k] < 0 || idx2[k] >= N) return -2;
    seg_csr(idx1, B, N, M, row_ptr1, col_idx1);
    seg_csr(idx2, B, M, N, row_ptr2, col_idx2);
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t p = 0; p < N; ++p) {
            int64_t r = b * N + p;
            const double* x = P + r * 3;
            const double* y = Q + (b * M + idx1[r]) * 3;
            for (int k = 0; k < 3; ++k) dP[r * 3 + k] = 2.0 * g1[r] * (x[k] - y[k]);
            for (int64_t e = row_ptr2[r]; e < row_ptr2[r + 1]; ++e) {
                int64_t q = col_idx2[e]; /* global index b*M + q */
                const double* z = Q + q * 3;
                for (int k = 0; k < 3; ++k) dP[r * 3 + k] += 2.0 * g2[q] * (x[k] - z[k]);
            }
        }
        for (int64_t q = 0; q < M; ++q) {
            int64_t r = b * M + q;
            const double* x = Q + r * 3;
            const double* y = P + (b * N + idx2[r]) * 3;
            for (int k = 0; k < 3; ++k) dQ[r * 3 + k] = 2.0 * g2[r] * (x[k] - y[k]);
            for (int64_t e = row_ptr1[r]; e < row_ptr1[r + 1]; ++e) {
                int64_t p = col_idx1[e];
                const double* z = P + p * 3;
                for (int k = 0; k < 3; ++k) dQ[r * 3 + k] += 2.0 * g1[p] * (x[k] - z[k]);
            }
        }
    }
    return 0;
}

int oracle_version(void) { return 4; }
