/*
 * fs_oracle.c -- plain fp64 CPU oracle of the FreeSolo FS-L attention forward.
 *
 * TEST INFRASTRUCTURE ONLY (see fs_oracle.h).  Written from the FreeSolo paper
 * summary (picx.dev page, "Methodology" sections 3.1-3.3).  Each query row is
 * evaluated on its own, in the order the equations are stated: no tiling, no
 * incremental state, no reuse across queries except the per-head cell
 * summaries, which eq. (5) defines per cell.
 */
#include "fs_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- RoPE (section 3.2, eq. 3; rotary embedding of Su et al.) ----------- */
void or_rope(const or_problem* p, const float* x, long long pos, double* out)
{
    const int d = p->head_dim;
    const double abs_pos = (double)(pos + p->pos_offset);
    for (int k = 0; k < d / 2; ++k) {
        const double theta = pow(p->rope_base, -2.0 * (double)k / (double)d);
        const double ang = abs_pos * theta;
        const double c = cos(ang), s = sin(ang);
        const double x0 = (double)x[2 * k], x1 = (double)x[2 * k + 1];
        out[2 * k] = x0 * c - x1 * s;
        out[2 * k + 1] = x0 * s + x1 * c;
    }
}

/* ---- candidate set C_i (eq. 6 is missing; complete cells ending before i-w) */
int or_n_candidates(const or_problem* p, long long i)
{
    if (i < p->window) return 0;
    long long n = (i - p->window) / p->cell;
    long long c_all = p->n_ctx / p->cell;
    return (int)(n < c_all ? n : c_all);
}

/* ---- cell summaries (section 3.3, eq. 5) ------------------------------- */
void or_cell_summaries_head(const or_problem* p, const float* k_head, double* kbar, double* amax)
{
    const int d = p->head_dim, s = p->cell, C = p->n_ctx / p->cell;
    for (int c = 0; c < C; ++c) {
        double* mean = kbar + (size_t)c * d;
        for (int e = 0; e < d; ++e) mean[e] = 0.0;
        double best = 0.0;
        for (int j = c * s; j < (c + 1) * s; ++j) {
            const float* kj = k_head + (size_t)j * d;
            double sq = 0.0;
            for (int e = 0; e < d; ++e) {
                mean[e] += (double)kj[e];
                sq += (double)kj[e] * (double)kj[e];
            }
            double norm = sqrt(sq);
            if (norm > best) best = norm;
        }
        for (int e = 0; e < d; ++e) mean[e] /= (double)s;
        amax[c] = best;
    }
}

/* ---- ordering helper: key descending, then cell index descending -------- */
typedef struct { double key; int cell; } or_keyed;

static int or_cmp_desc(const void* a, const void* b)
{
    const or_keyed* x = (const or_keyed*)a;
    const or_keyed* y = (const or_keyed*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    if (x->cell > y->cell) return -1;
    if (x->cell < y->cell) return 1;
    return 0;
}

static double or_rel_gap(double hi, double lo)
{
    double den = fabs(hi) > fabs(lo) ? fabs(hi) : fabs(lo);
    if (den == 0.0) return 0.0;
    return (hi - lo) / den;
}

static int or_cmp_int(const void* a, const void* b)
{
    int x = *(const int*)a, y = *(const int*)b;
    return (x > y) - (x < y);
}

/* ---- FS-L query-independent pruning (section 3.3, eq. 8) --------------- */
int or_prune_row(const or_problem* p, const double* amax, int n, int* keep, double* gap_rel)
{
    if (gap_rel) *gap_rel = INFINITY;
    if (n <= 0) return 0;
    if (p->budget < 0) {                     /* no pruning: A_i = C_i */
        for (int c = 0; c < n; ++c) keep[c] = c;
        return n;
    }
    or_keyed* order = (or_keyed*)malloc(sizeof(or_keyed) * (size_t)n);
    unsigned char* kept = (unsigned char*)calloc((size_t)n, 1);
    for (int c = 0; c < n; ++c) { order[c].key = amax[c]; order[c].cell = c; }
    qsort(order, (size_t)n, sizeof(or_keyed), or_cmp_desc);
    /* TopP over C_i by norm priority a_c */
    for (int r = 0; r < n && r < p->budget; ++r) kept[order[r].cell] = 1;
    if (gap_rel && p->budget > 0 && n > p->budget)
        *gap_rel = or_rel_gap(order[p->budget - 1].key, order[p->budget].key);
    /* Recent_W: the W most recent candidate cells */
    for (int c = n - p->n_recent; c < n; ++c)
        if (c >= 0) kept[c] = 1;
    int cnt = 0;
    for (int c = 0; c < n; ++c)
        if (kept[c]) keep[cnt++] = c;
    free(order);
    free(kept);
    return cnt;
}

/* ---- query-dependent scoring and top-K (eq. 7 with lambda_h = 0) ------- */
/* ---- eq. 7's position prior ------------------------------------------ */
double or_prior(const or_problem* p, int head, long long i, int c, double a_c)
{
    if (!p->prior_lambda || !p->prior_sigma || head < 0) return 0.0;
    const double lam = p->prior_lambda[head], sig = p->prior_sigma[head];
    const double p_c = ((double)c + 0.5) * (double)p->cell;       /* eq. 5 */
    return lam * a_c * erf(((double)i - p_c) / (2.0 * sig));
}

int or_select_row_at(const or_problem* p, int head, long long i, const float* q_row,
                     const double* kbar, const double* amax, const int* cand, int n_cand,
                     int* sel, double* gap_rel, double* cand_scores)
{
    const int d = p->head_dim;
    if (gap_rel) *gap_rel = INFINITY;
    if (n_cand <= 0) return 0;
    or_keyed* order = (or_keyed*)malloc(sizeof(or_keyed) * (size_t)n_cand);
    for (int t = 0; t < n_cand; ++t) {
        const double* kb = kbar + (size_t)cand[t] * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += (double)q_row[e] * kb[e];
        order[t].key = dot / sqrt((double)d) +
                       (amax ? or_prior(p, head, i, cand[t], amax[cand[t]]) : 0.0);
        order[t].cell = cand[t];
        if (cand_scores) cand_scores[t] = order[t].key;
    }
    qsort(order, (size_t)n_cand, sizeof(or_keyed), or_cmp_desc);
    int cnt = n_cand < p->topk ? n_cand : p->topk;
    if (gap_rel && n_cand > p->topk && p->topk > 0)
        *gap_rel = or_rel_gap(order[p->topk - 1].key, order[p->topk].key);
    for (int t = 0; t < cnt; ++t) sel[t] = order[t].cell;
    qsort(sel, (size_t)cnt, sizeof(int), or_cmp_int);
    free(order);
    return cnt;
}

/* ---- token-level reranking (section 3.4, eq. 12) ---------------------- */
static double or_cell_lse(const or_problem* p, const float* q_row, const float* k_head, int c)
{
    const int d = p->head_dim, s = p->cell;
    double* lg = (double*)malloc(sizeof(double) * (size_t)s);
    double mx = -INFINITY;
    for (int t = 0; t < s; ++t) {
        const float* kj = k_head + ((size_t)c * s + t) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += (double)q_row[e] * (double)kj[e];
        lg[t] = dot / sqrt((double)d);
        if (lg[t] > mx) mx = lg[t];
    }
    double sum = 0.0;
    for (int t = 0; t < s; ++t) sum += exp(lg[t] - mx);
    free(lg);
    return mx + log(sum);
}

int or_rerank_row(const or_problem* p, int head, long long i, const float* q_row,
                  const float* k_head, const double* amax, const int* cand, int n_cand,
                  int* sel, double* gap_rel, double* cand_scores)
{
    if (gap_rel) *gap_rel = INFINITY;
    if (n_cand <= 0) return 0;
    or_keyed* order = (or_keyed*)malloc(sizeof(or_keyed) * (size_t)n_cand);
    for (int t = 0; t < n_cand; ++t) {
        order[t].key = or_cell_lse(p, q_row, k_head, cand[t]) +
                       (amax ? or_prior(p, head, i, cand[t], amax[cand[t]]) : 0.0);
        order[t].cell = cand[t];
        if (cand_scores) cand_scores[t] = order[t].key;
    }
    qsort(order, (size_t)n_cand, sizeof(or_keyed), or_cmp_desc);
    int cnt = n_cand < p->topk ? n_cand : p->topk;
    if (gap_rel && n_cand > p->topk && p->topk > 0)
        *gap_rel = or_rel_gap(order[p->topk - 1].key, order[p->topk].key);
    for (int t = 0; t < cnt; ++t) sel[t] = order[t].cell;
    qsort(sel, (size_t)cnt, sizeof(int), or_cmp_int);
    free(order);
    return cnt;
}

int or_select_row(const or_problem* p, const float* q_row, const double* kbar,
                  const int* cand, int n_cand, int* sel, double* gap_rel, double* cand_scores)
{
    return or_select_row_at(p, -1, 0, q_row, kbar, NULL, cand, n_cand, sel, gap_rel,
                            cand_scores);
}

/* ---- softmax-weighted sum of value rows over a list of token positions -- */
static void or_attend(int d, const double* logits, const int* tok, int n_tok,
                      const float* v_head, double* out)
{
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    if (n_tok <= 0) return;
    double mx = logits[0];
    for (int t = 1; t < n_tok; ++t)
        if (logits[t] > mx) mx = logits[t];
    double den = 0.0;
    for (int t = 0; t < n_tok; ++t) den += exp(logits[t] - mx);
    for (int t = 0; t < n_tok; ++t) {
        const double w = exp(logits[t] - mx) / den;
        const float* vj = v_head + (size_t)tok[t] * d;
        for (int e = 0; e < d; ++e) out[e] += w * (double)vj[e];
    }
}

/* ---- local branch (section 3.2, eqs. 3-4) ------------------------------ */
void or_window_row(const or_problem* p, const float* q_row, const float* k_head,
                   const float* v_head, long long i, double* o_sr)
{
    const int d = p->head_dim;
    long long lo = i - p->window;
    if (lo < 0) lo = 0;
    const int n_tok = (int)(i - lo + 1);
    double* rq = (double*)malloc(sizeof(double) * (size_t)d);
    double* rk = (double*)malloc(sizeof(double) * (size_t)d);
    double* logits = (double*)malloc(sizeof(double) * (size_t)n_tok);
    int* tok = (int*)malloc(sizeof(int) * (size_t)n_tok);
    or_rope(p, q_row, i, rq);
    for (int t = 0; t < n_tok; ++t) {
        const long long j = lo + t;
        or_rope(p, k_head + (size_t)j * d, j, rk);
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += rq[e] * rk[e];
        logits[t] = dot / sqrt((double)d);
        tok[t] = (int)j;
    }
    or_attend(d, logits, tok, n_tok, v_head, o_sr);
    free(rq); free(rk); free(logits); free(tok);
}

/* ---- long-range readout with RMSNorm (section 3.3, eq. 9) -------------- */
void or_sparse_row(const or_problem* p, const float* q_row, const float* k_head,
                   const float* v_head, const int* sel, int n_sel, double* o_lr)
{
    const int d = p->head_dim, s = p->cell;
    const int n_tok = n_sel * s;
    for (int e = 0; e < d; ++e) o_lr[e] = 0.0;
    if (n_tok == 0) return;                  /* empty T_i: u = 0, so o_lr = 0 */
    double* logits = (double*)malloc(sizeof(double) * (size_t)n_tok);
    int* tok = (int*)malloc(sizeof(int) * (size_t)n_tok);
    double* u = (double*)malloc(sizeof(double) * (size_t)d);
    int t = 0;
    for (int a = 0; a < n_sel; ++a) {
        for (int j = sel[a] * s; j < (sel[a] + 1) * s; ++j) {
            const float* kj = k_head + (size_t)j * d;
            double dot = 0.0;
            for (int e = 0; e < d; ++e) dot += (double)q_row[e] * (double)kj[e];
            logits[t] = dot / sqrt((double)d);
            tok[t] = j;
            ++t;
        }
    }
    or_attend(d, logits, tok, n_tok, v_head, u);
    double ms = 0.0;
    for (int e = 0; e < d; ++e) ms += u[e] * u[e];
    ms /= (double)d;
    const double inv = 1.0 / sqrt(ms + p->rms_eps);
    for (int e = 0; e < d; ++e) o_lr[e] = u[e] * inv;
    free(logits); free(tok); free(u);
}

/* ---- one query row of the whole forward (eq. 2) ------------------------ */
static void or_forward_one(const or_problem* p, int head, const float* q_row,
                           const float* k_head, const float* v_head, const double* kbar,
                           const double* amax, double alpha, long long i,
                           const int* keep_ovr, int keep_ovr_n,
                           const int* sel_ovr, int sel_ovr_n,
                           double* o, double* o_sr, double* o_lr,
                           int* sel, int* n_sel, double* sel_gap, double* keep_gap)
{
    const int d = p->head_dim;
    or_window_row(p, q_row, k_head, v_head, i, o_sr);

    const int n = or_n_candidates(p, i);
    int* keep = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    int n_keep;
    double kg = INFINITY, sg = INFINITY;
    if (keep_ovr && keep_ovr_n >= 0) {
        n_keep = keep_ovr_n;
        keep = (int*)realloc(keep, sizeof(int) * (size_t)(n_keep > 0 ? n_keep : 1));
        memcpy(keep, keep_ovr, sizeof(int) * (size_t)n_keep);
    } else {
        n_keep = or_prune_row(p, amax, n, keep, &kg);
    }
    const int cap = p->topk > 0 ? p->topk : 1;
    int* chosen = (int*)malloc(sizeof(int) * (size_t)(n_keep > cap ? n_keep : cap));
    int n_chosen;
    if (sel_ovr && sel_ovr_n >= 0) {
        n_chosen = sel_ovr_n;
        memcpy(chosen, sel_ovr, sizeof(int) * (size_t)n_chosen);
    } else {
        n_chosen = or_select_row_at(p, head, i, q_row, kbar, amax, keep, n_keep, chosen, &sg,
                                    NULL);
    }
    or_sparse_row(p, q_row, k_head, v_head, chosen, n_chosen, o_lr);
    for (int e = 0; e < d; ++e) o[e] = o_sr[e] + alpha * o_lr[e];
    if (sel) {
        for (int t = 0; t < p->topk; ++t) sel[t] = t < n_chosen ? chosen[t] : -1;
    }
    if (n_sel) *n_sel = n_chosen;
    if (sel_gap) *sel_gap = sg;
    if (keep_gap) *keep_gap = kg;
    free(keep);
    free(chosen);
}

/* ---- thread pool over query rows ---------------------------------------- */
typedef struct {
    const or_problem* p;
    const float *q_head, *k_head, *v_head;
    const double *kbar, *amax;
    double alpha;
    const int* rows;
    int n_rows;
    const int *keep_ovr, *keep_ovr_n;
    int keep_w;
    const int *sel_ovr, *sel_ovr_n;
    double *o, *o_sr, *o_lr;
    int *sel, *n_sel;
    double *sel_gap, *keep_gap;
    int head;
    int next;                      /* shared work counter */
    pthread_mutex_t lock;
} or_rows_job;

static void* or_rows_worker(void* arg)
{
    or_rows_job* J = (or_rows_job*)arg;
    const int d = J->p->head_dim;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int r = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->n_rows) break;
        const int t = J->rows[r];
        const long long i = (long long)J->p->q_pos0 + t;
        or_forward_one(J->p, J->head, J->q_head + (size_t)t * d, J->k_head, J->v_head, J->kbar,
                       J->amax, J->alpha, i,
                       J->keep_ovr ? J->keep_ovr + (size_t)r * J->keep_w : NULL,
                       J->keep_ovr_n ? J->keep_ovr_n[r] : -1,
                       J->sel_ovr ? J->sel_ovr + (size_t)r * J->p->topk : NULL,
                       J->sel_ovr_n ? J->sel_ovr_n[r] : -1,
                       J->o + (size_t)r * d, J->o_sr + (size_t)r * d, J->o_lr + (size_t)r * d,
                       J->sel ? J->sel + (size_t)r * J->p->topk : NULL,
                       J->n_sel ? J->n_sel + r : NULL,
                       J->sel_gap ? J->sel_gap + r : NULL,
                       J->keep_gap ? J->keep_gap + r : NULL);
    }
    return NULL;
}

int or_forward_rows(const or_problem* p, const float* q_head, const float* k_head,
                    const float* v_head, const double* kbar, const double* amax,
                    double alpha, const int* rows, int n_rows,
                    const int* keep_ovr, const int* keep_ovr_n, int keep_w,
                    const int* sel_ovr, const int* sel_ovr_n,
                    double* o, double* o_sr, double* o_lr, int* sel, int* n_sel,
                    double* sel_gap, double* keep_gap, int nthreads, int head)
{
    or_rows_job J;
    memset(&J, 0, sizeof(J));
    J.p = p; J.q_head = q_head; J.k_head = k_head; J.v_head = v_head;
    J.kbar = kbar; J.amax = amax; J.alpha = alpha; J.rows = rows; J.n_rows = n_rows;
    J.keep_ovr = keep_ovr; J.keep_ovr_n = keep_ovr_n; J.keep_w = keep_w;
    J.sel_ovr = sel_ovr; J.sel_ovr_n = sel_ovr_n;
    J.o = o; J.o_sr = o_sr; J.o_lr = o_lr; J.sel = sel; J.n_sel = n_sel;
    J.sel_gap = sel_gap; J.keep_gap = keep_gap; J.head = head;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int t = 0; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, or_rows_worker, &J) == 0) ++started;
    if (started == 0) or_rows_worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

int or_forward(const or_problem* p, const float* q, const float* k, const float* v,
               const float* alpha, double* o, double* o_sr, double* o_lr,
               int* sel, int* n_sel, double* sel_gap, double* keep_gap, int nthreads)
{
    const int d = p->head_dim, N = p->n_ctx, C = p->n_ctx / p->cell, nq = p->n_q;
    double* kbar = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1) * d);
    double* amax = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    int* rows = (int*)malloc(sizeof(int) * (size_t)(nq > 0 ? nq : 1));
    for (int t = 0; t < nq; ++t) rows[t] = t;
    for (int b = 0; b < p->batch; ++b) {
        for (int h = 0; h < p->heads; ++h) {
            const size_t bh = (size_t)b * p->heads + h;
            const float* kh = k + bh * (size_t)N * d;
            const float* vh = v + bh * (size_t)N * d;
            const float* qh = q + bh * (size_t)nq * d;
            or_cell_summaries_head(p, kh, kbar, amax);
            or_forward_rows(p, qh, kh, vh, kbar, amax, (double)alpha[h], rows, nq,
                            NULL, NULL, 0, NULL, NULL,
                            o + bh * (size_t)nq * d, o_sr + bh * (size_t)nq * d,
                            o_lr + bh * (size_t)nq * d,
                            sel ? sel + bh * (size_t)nq * p->topk : NULL,
                            n_sel ? n_sel + bh * (size_t)nq : NULL,
                            sel_gap ? sel_gap + bh * (size_t)nq : NULL,
                            keep_gap ? keep_gap + bh * (size_t)nq : NULL, nthreads, h);
        }
    }
    free(kbar); free(amax); free(rows);
    return 0;
}
