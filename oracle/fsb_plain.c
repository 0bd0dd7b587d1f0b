/*
 * fsb_plain.c -- plain fp64 CPU oracle of FreeSolo's balanced tree search (FS-B).
 *
 * TEST INFRASTRUCTURE ONLY (see fs_oracle.h).  Written from the FreeSolo paper
 * summary (picx.dev page), section 3.4 "Balanced Tree Search (FS-B)": the
 * admitted sets of eq. (10), the node utility U_v of eq. (11), and eq. (7)'s
 * score over the leaves the search finds.  It takes the same readings of what
 * the page leaves open as fsb_oracle.c (forests of complete aligned
 * power-of-two blocks; mu_v the mean of the node's cell means, rho_v the
 * largest distance from mu_v to one of them, A_v the largest a_c, p_v^min the
 * centre of the first cell; a beam of width B per forest that expands every
 * inner node and keeps the best B; S_i the best K found leaves; ties to the
 * larger U, then the later block, then the lower level), but computes
 * everything in plain fp64 from the fp64 cell summaries of eq. (5):
 *   - node statistics are fp64 sums and distances, never rounded to float;
 *   - dot products run over the d components in index order;
 *   - U_v = (q . mu_v + c |q| rho_v) / sqrt(d) + lambda_h A_v erf((i - p_v^min) / (2 sigma_h)).
 * It shares nothing with fsb_oracle.c, whose arithmetic fixes one reduction
 * order and float32 node statistics.  Each search records the smallest
 * relative gap at which it decided between two entries (the B-th and
 * (B+1)-th U of every cut, and the K-th and (K+1)-th score of the final
 * top-K): a row whose gap is below a tolerance may legitimately come out
 * differently under another rounding.
 */
#include "fs_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

static int pl_floor_log2(int m)
{
    int l = 0;
    while ((2 << l) <= m) ++l;
    return l;
}

int or_forest64_build(const double* kbar, const double* amax, int n_cells, int d, int use_tau,
                      double tau, or_forest64* f)
{
    f->n_cells = n_cells;
    f->head_dim = d;
    int m = 0;
    f->prefix[0] = 0;
    for (int c = 0; c < n_cells; ++c) {
        if (!use_tau || amax[c] >= tau) f->cell_of[m++] = c;   /* eq. 10: a_c >= tau */
        f->prefix[c + 1] = m;
    }
    f->m = m;
    f->n_levels = m > 0 ? pl_floor_log2(m) + 1 : 0;
    int start = 0;
    for (int l = 0; l < f->n_levels; ++l) {
        f->level_start[l] = start;
        start += m >> l;
    }
    for (int l = 0; l < f->n_levels; ++l) {
        const int width = 1 << l;
        for (int j = 0; j < (m >> l); ++j) {
            const int node = f->level_start[l] + j;
            double* mu = f->mu + (size_t)node * d;
            double a_best = -INFINITY;
            for (int e = 0; e < d; ++e) mu[e] = 0.0;
            for (int t = 0; t < width; ++t) {
                const int c = f->cell_of[j * width + t];
                for (int e = 0; e < d; ++e) mu[e] += kbar[(size_t)c * d + e];
                if (amax[c] > a_best) a_best = amax[c];
            }
            for (int e = 0; e < d; ++e) mu[e] /= (double)width;
            double r2 = 0.0;
            for (int t = 0; t < width; ++t) {
                const int c = f->cell_of[j * width + t];
                double acc = 0.0;
                for (int e = 0; e < d; ++e) {
                    const double diff = kbar[(size_t)c * d + e] - mu[e];
                    acc += diff * diff;
                }
                if (acc > r2) r2 = acc;
            }
            f->rho[node] = sqrt(r2);
            f->amax[node] = a_best;
            f->first[node] = f->cell_of[j * width];
        }
    }
    return m;
}

/* U_v of node (level, index), eq. 11. */
double or_node64_score(const or_problem* p, int head, long long i, const float* q_row,
                       const or_forest64* f, int level, int index, double slack)
{
    const int d = p->head_dim;
    const int node = f->level_start[level] + index;
    const double* mu = f->mu + (size_t)node * d;
    double dot = 0.0, qq = 0.0;
    for (int e = 0; e < d; ++e) {
        dot += (double)q_row[e] * mu[e];
        qq += (double)q_row[e] * (double)q_row[e];
    }
    const double u = (dot + slack * sqrt(qq) * f->rho[node]) / sqrt((double)d);
    return u + or_prior(p, head, i, f->first[node], f->amax[node]);
}

typedef struct {
    double u;
    int level, index, first;
} pl_ent;

/* larger U first; then the later block; then the lower level */
static int pl_cmp(const void* a, const void* b)
{
    const pl_ent* x = (const pl_ent*)a;
    const pl_ent* y = (const pl_ent*)b;
    if (x->u != y->u) return x->u > y->u ? -1 : 1;
    if (x->first != y->first) return x->first > y->first ? -1 : 1;
    return x->level < y->level ? -1 : (x->level > y->level ? 1 : 0);
}

static double pl_rel_gap(double a, double b)
{
    const double s = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
    return s > 0.0 ? fabs(a - b) / s : INFINITY;
}

/* Keep the best `keep` of n sorted entries; note the gap at the cut. */
static int pl_cut(pl_ent* e, int n, int keep, double* gap)
{
    qsort(e, (size_t)n, sizeof(pl_ent), pl_cmp);
    if (n <= keep) return n;
    const double g = pl_rel_gap(e[keep - 1].u, e[keep].u);
    if (g < *gap) *gap = g;
    return keep;
}

/* Roots covering the first n leaves: one per set bit of n, largest first. */
int or_forest64_roots(const or_forest64* f, int n, int* level, int* index)
{
    int cnt = 0, start = 0;
    for (int l = f->n_levels - 1; l >= 0; --l)
        if ((n >> l) & 1) {
            level[cnt] = l;
            index[cnt] = start >> l;
            ++cnt;
            start += 1 << l;
        }
    return cnt;
}

static int pl_beam_forest(const or_problem* p, int head, long long i, const float* q,
                          const or_forest64* f, int n_leaves, int beam, double slack,
                          pl_ent* found, int* n_scored, double* gap)
{
    if (!f || n_leaves <= 0 || beam <= 0) return 0;
    pl_ent* cur = (pl_ent*)malloc(sizeof(pl_ent) * (size_t)(2 * beam + 32));
    pl_ent* cand = (pl_ent*)malloc(sizeof(pl_ent) * (size_t)(2 * beam + 32));
    int lv[32], ix[32];
    const int n_roots = or_forest64_roots(f, n_leaves, lv, ix);
    for (int r = 0; r < n_roots; ++r) {
        cur[r].level = lv[r];
        cur[r].index = ix[r];
        cur[r].first = f->first[f->level_start[lv[r]] + ix[r]];
        cur[r].u = or_node64_score(p, head, i, q, f, lv[r], ix[r], slack);
    }
    *n_scored += n_roots;
    int n_cur = pl_cut(cur, n_roots, beam, gap);
    for (;;) {
        int n_cand = 0, inner = 0;
        for (int t = 0; t < n_cur; ++t) {
            if (cur[t].level == 0) {
                cand[n_cand++] = cur[t];
                continue;
            }
            inner = 1;
            for (int ch = 0; ch < 2; ++ch) {
                pl_ent e;
                e.level = cur[t].level - 1;
                e.index = 2 * cur[t].index + ch;
                e.first = f->first[f->level_start[e.level] + e.index];
                e.u = or_node64_score(p, head, i, q, f, e.level, e.index, slack);
                cand[n_cand++] = e;
                ++*n_scored;
            }
        }
        if (!inner) break;
        n_cur = pl_cut(cand, n_cand, beam, gap);
        pl_ent* t = cur;
        cur = cand;
        cand = t;
    }
    memcpy(found, cur, sizeof(pl_ent) * (size_t)n_cur);
    free(cur);
    free(cand);
    return n_cur;
}

/* The leaves both searches end with, without repeats (a cell found by both
 * forests has one score), in search order; *gap receives the smallest relative
 * gap of the searches' cuts. */
static int pl_found(const or_problem* p, int head, long long i, const float* q_row,
                    const or_forest64* f0, const or_forest64* ftau, int beam, double slack,
                    pl_ent* found, int* n_scored, double* gap)
{
    int scored = 0;
    const int n = or_n_candidates(p, i);
    int cnt = 0;
    if (f0)
        cnt += pl_beam_forest(p, head, i, q_row, f0, f0->prefix[n < f0->n_cells ? n : f0->n_cells],
                              beam, slack, found, &scored, gap);
    if (ftau)
        cnt += pl_beam_forest(p, head, i, q_row, ftau,
                              ftau->prefix[n < ftau->n_cells ? n : ftau->n_cells], beam, slack,
                              found + cnt, &scored, gap);
    int n_u = 0;
    for (int t = 0; t < cnt; ++t) {
        int dup = 0;
        for (int r = 0; r < n_u; ++r) dup |= found[r].first == found[t].first;
        if (!dup) found[n_u++] = found[t];
    }
    if (n_scored) *n_scored = scored;
    return n_u;
}

int or_beam64_found(const or_problem* p, int head, long long i, const float* q_row,
                    const or_forest64* f0, const or_forest64* ftau, int beam, double slack,
                    int* cells, int* n_scored, double* gap)
{
    double g = INFINITY;
    pl_ent* found = (pl_ent*)malloc(sizeof(pl_ent) * (size_t)(2 * beam + 2));
    const int n_u = pl_found(p, head, i, q_row, f0, ftau, beam, slack, found, n_scored, &g);
    for (int t = 0; t < n_u; ++t) cells[t] = found[t].first;
    free(found);
    if (gap) *gap = g;
    return n_u;
}

int or_beam64_row(const or_problem* p, int head, long long i, const float* q_row,
                  const or_forest64* f0, const or_forest64* ftau, int beam, double slack,
                  int* sel, double* score, int* n_scored, double* gap)
{
    double g = INFINITY;
    pl_ent* found = (pl_ent*)malloc(sizeof(pl_ent) * (size_t)(2 * beam + 2));
    const int n_u = pl_found(p, head, i, q_row, f0, ftau, beam, slack, found, n_scored, &g);
    /* eq. 7's score of a leaf is its U: the best K of the found cells */
    const int k = pl_cut(found, n_u, p->topk, &g);
    for (int t = 0; t < k; ++t) {
        sel[t] = found[t].first;
        if (score) score[t] = found[t].u;
    }
    free(found);
    if (gap) *gap = g;
    return k;
}

/* ---- many rows of one head, threaded ------------------------------------ */
typedef struct {
    const or_problem* p;
    int head;
    const float* q_head;
    const int* rows;
    int n_rows;
    const or_forest64 *f0, *ftau;
    int beam;
    double slack;
    int* sel;
    double* score;
    int* n_sel;
    int* n_scored;
    double* gap;
    int next;
    pthread_mutex_t lock;
} pl_job;

static void* pl_worker(void* arg)
{
    pl_job* J = (pl_job*)arg;
    const int K = J->p->topk, d = J->p->head_dim;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int r = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->n_rows) break;
        const int t = J->rows[r];
        int* s = J->sel + (size_t)r * K;
        double* sc = J->score + (size_t)r * K;
        for (int e = 0; e < K; ++e) {
            s[e] = -1;
            sc[e] = 0.0;
        }
        J->n_sel[r] = or_beam64_row(J->p, J->head, (long long)J->p->q_pos0 + t,
                                    J->q_head + (size_t)t * d, J->f0, J->ftau, J->beam, J->slack,
                                    s, sc, J->n_scored + r, J->gap + r);
    }
    return NULL;
}

int or_beam64_rows(const or_problem* p, int head, const float* q_head, const int* rows,
                   int n_rows, const or_forest64* f0, const or_forest64* ftau, int beam,
                   double slack, int* sel, double* score, int* n_sel, int* n_scored,
                   double* gap, int nthreads)
{
    pl_job J = {p, head, q_head, rows, n_rows, f0, ftau, beam, slack, sel, score, n_sel,
                n_scored, gap, 0};
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int t = 0; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, pl_worker, &J) == 0) ++started;
    if (started == 0) pl_worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return 0;
}
