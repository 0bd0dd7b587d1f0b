/*
 * fsb_oracle.c -- plain CPU oracle of FreeSolo's balanced tree search (FS-B).
 *
 * TEST INFRASTRUCTURE ONLY (see fs_oracle.h).  Written from the FreeSolo paper
 * summary (picx.dev page), section 3.4 "Balanced Tree Search (FS-B)", eqs. (10)
 * and (11), with eq. (5)'s cell summaries and eq. (7)'s cell score.  The page
 * gives the admitted sets and the node score but not the forest, the node
 * statistics or the search; the readings taken here are:
 *   - a causal forest over a sequence of cells is the set of complete,
 *     aligned power-of-two blocks of that sequence.  Node (l, j) covers leaves
 *     j 2^l .. (j+1) 2^l - 1, and its children are (l-1, 2j) and (l-1, 2j+1).
 *     A prefix of n leaves is covered by one root per set bit of n, largest
 *     first.  A block never changes once complete, so the forest grows with
 *     the archive;
 *   - forest 0 holds every complete cell (A^0 = C_i).  Forest tau holds the
 *     cells with a_c >= tau_h, in ascending order (A^tau, eq. 10).  Query i
 *     searches the prefix of each forest that lies in C_i;
 *   - mu_v is the mean of the node's cell means, rho_v the largest distance
 *     from mu_v to one of them, A_v the largest a_c, and p_v^min the centre of
 *     the node's first cell.  With slack c = 1 and lambda_h >= 0, U_v is then
 *     an upper bound of the eq. (7) score of every cell below v;
 *   - beam search: start from the roots (the best B of them).  Each step
 *     replaces every internal node of the beam by its two children, keeps
 *     leaves, and retains the best B by U.  It stops when the beam holds
 *     leaves only.  A leaf's U equals eq. (7)'s r_ic;
 *   - S_i is the best min(K, |leaves|) of the union of the two final beams by
 *     r_ic.  Ties go to the larger cell index; between inner nodes of equal
 *     U, the later block wins, then the lower level.
 * The search decides by comparing U values, so the oracle computes them in
 * the kernel's precision and order: fp64 arithmetic on the fp32 node
 * statistics, a dot product as 16 partial sums over contiguous d/16-element
 * chunks added by the butterfly (pairs at distance 8, 4, 2, 1), and the node
 * statistics from sums in ascending leaf order.  Built with fp contraction
 * off.
 */
#include "fs_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- dot product in the fixed order described above --------------------- */
double or_dot16(const float* a, const float* b, int d)
{
    const int chunk = d / 16;
    double part[16], next[16];
    for (int t = 0; t < 16; ++t) {
        double acc = 0.0;
        for (int u = 0; u < chunk; ++u)
            acc = fma((double)a[t * chunk + u], (double)b[t * chunk + u], acc);
        part[t] = acc;
    }
    for (int off = 8; off >= 1; off >>= 1) {
        for (int t = 0; t < 16; ++t) next[t] = part[t] + part[t ^ off];
        memcpy(part, next, sizeof(part));
    }
    return part[0];
}

static int or_floor_log2(int m)
{
    int l = 0;
    while ((2 << l) <= m) ++l;
    return l;
}

/* ---- forest construction (eq. 10 admitted set, node statistics) -------- */
int or_forest_build(const float* kbar, const float* amax, int n_cells, int d, int use_tau,
                    double tau, or_forest* f)
{
    f->n_cells = n_cells;
    f->head_dim = d;
    int m = 0;
    f->prefix[0] = 0;
    for (int c = 0; c < n_cells; ++c) {
        if (!use_tau || (double)amax[c] >= tau) f->cell_of[m++] = c;
        f->prefix[c + 1] = m;
    }
    f->m = m;
    f->n_levels = m > 0 ? or_floor_log2(m) + 1 : 0;
    int start = 0;
    for (int l = 0; l < f->n_levels; ++l) {
        f->level_start[l] = start;
        start += m >> l;
    }
    double* sum = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
    for (int l = 0; l < f->n_levels; ++l) {
        const int width = 1 << l;
        for (int j = 0; j < (m >> l); ++j) {
            const int node = f->level_start[l] + j;
            const int leaf0 = j * width;
            float* mu = f->mu + (size_t)node * d;
            /* mean of the cell means, summed in ascending leaf order */
            for (int e = 0; e < d; ++e) sum[e] = 0.0;
            float a_best = -INFINITY;
            for (int t = 0; t < width; ++t) {
                const int c = f->cell_of[leaf0 + t];
                for (int e = 0; e < d; ++e) sum[e] += (double)kbar[(size_t)c * d + e];
                if (amax[c] > a_best) a_best = amax[c];
            }
            for (int e = 0; e < d; ++e) mu[e] = (float)(sum[e] * ldexp(1.0, -l));
            /* largest distance from mu to a cell mean below the node */
            double r2 = 0.0;
            for (int t = 0; t < width; ++t) {
                const int c = f->cell_of[leaf0 + t];
                double acc = 0.0;
                for (int e = 0; e < d; ++e) {
                    const double diff = (double)kbar[(size_t)c * d + e] - (double)mu[e];
                    acc = fma(diff, diff, acc);
                }
                if (acc > r2) r2 = acc;
            }
            f->rho[node] = (float)sqrt(r2);
            f->amax[node] = a_best;
            f->first[node] = f->cell_of[leaf0];
        }
    }
    free(sum);
    return m;
}

int or_forest_roots(const or_forest* f, int n_leaves, int* level, int* index)
{
    int cnt = 0, start = 0;
    for (int l = f->n_levels - 1; l >= 0; --l) {
        if ((n_leaves >> l) & 1) {
            level[cnt] = l;
            index[cnt] = start >> l;
            ++cnt;
            start += 1 << l;
        }
    }
    return cnt;
}

/* ---- node score U_v (eq. 11) ------------------------------------------- */
double or_node_score(const or_problem* p, int head, long long i, const float* q_row,
                     double q_norm, const or_forest* f, int level, int index, double slack)
{
    const int d = p->head_dim;
    const int node = f->level_start[level] + index;
    const double dot = or_dot16(q_row, f->mu + (size_t)node * d, d);
    double t = slack * q_norm;
    t = t * (double)f->rho[node];
    double u = dot + t;
    u = u * (1.0 / sqrt((double)d));
    /* lambda_h A_v g_h(i - p_v^min): eq. 7's prior at the node's first cell */
    return u + or_prior(p, head, i, f->first[node], (double)f->amax[node]);
}

typedef struct {
    double u;
    int level, index, first;
} or_beam_ent;

/* larger U first; then the later block; then the lower level */
static int or_cmp_beam(const void* a, const void* b)
{
    const or_beam_ent* x = (const or_beam_ent*)a;
    const or_beam_ent* y = (const or_beam_ent*)b;
    if (x->u > y->u) return -1;
    if (x->u < y->u) return 1;
    if (x->first > y->first) return -1;
    if (x->first < y->first) return 1;
    return x->level < y->level ? -1 : (x->level > y->level ? 1 : 0);
}

/* Beam search of one forest over its first n_leaves leaves.  Writes the final
 * beam's cells and scores; returns their count. */
static int or_beam_forest(const or_problem* p, int head, long long i, const float* q_row,
                          double q_norm, const or_forest* f, int n_leaves, int beam,
                          double slack, int* cells, double* scores, int* n_scored)
{
    if (!f || n_leaves <= 0 || beam <= 0) return 0;
    or_beam_ent* cur = (or_beam_ent*)malloc(sizeof(or_beam_ent) * (size_t)(2 * beam + 32));
    or_beam_ent* cand = (or_beam_ent*)malloc(sizeof(or_beam_ent) * (size_t)(2 * beam + 32));
    int lv[32], ix[32];
    const int n_roots = or_forest_roots(f, n_leaves, lv, ix);
    int n_cur = 0;
    for (int r = 0; r < n_roots; ++r) {
        cur[n_cur].level = lv[r];
        cur[n_cur].index = ix[r];
        cur[n_cur].first = f->first[f->level_start[lv[r]] + ix[r]];
        cur[n_cur].u = or_node_score(p, head, i, q_row, q_norm, f, lv[r], ix[r], slack);
        ++n_cur;
        ++*n_scored;
    }
    qsort(cur, (size_t)n_cur, sizeof(or_beam_ent), or_cmp_beam);
    if (n_cur > beam) n_cur = beam;
    for (;;) {
        int inner = 0;
        for (int t = 0; t < n_cur; ++t) inner |= cur[t].level > 0;
        if (!inner) break;
        int n_cand = 0;
        for (int t = 0; t < n_cur; ++t) {
            if (cur[t].level == 0) {
                cand[n_cand++] = cur[t];
                continue;
            }
            for (int ch = 0; ch < 2; ++ch) {
                or_beam_ent e;
                e.level = cur[t].level - 1;
                e.index = 2 * cur[t].index + ch;
                e.first = f->first[f->level_start[e.level] + e.index];
                e.u = or_node_score(p, head, i, q_row, q_norm, f, e.level, e.index, slack);
                cand[n_cand++] = e;
                ++*n_scored;
            }
        }
        qsort(cand, (size_t)n_cand, sizeof(or_beam_ent), or_cmp_beam);
        n_cur = n_cand < beam ? n_cand : beam;
        memcpy(cur, cand, sizeof(or_beam_ent) * (size_t)n_cur);
    }
    for (int t = 0; t < n_cur; ++t) {
        cells[t] = cur[t].first;
        scores[t] = cur[t].u;
    }
    free(cur);
    free(cand);
    return n_cur;
}

/* ---- S_i of one query (eqs. 10-11, then eq. 7 over the found leaves) ----- */
int or_beam_row(const or_problem* p, int head, long long i, const float* q_row,
                const or_forest* f0, const or_forest* ftau, int beam, double slack,
                int* sel, double* score, int* n_scored)
{
    int scored = 0;
    const int d = p->head_dim;
    const int n = or_n_candidates(p, i);
    const double q_norm = sqrt(or_dot16(q_row, q_row, d));
    int* cells = (int*)malloc(sizeof(int) * (size_t)(2 * beam + 2));
    double* sc = (double*)malloc(sizeof(double) * (size_t)(2 * beam + 2));
    int cnt = 0;
    if (f0) cnt += or_beam_forest(p, head, i, q_row, q_norm, f0,
                                  f0->prefix[n < f0->n_cells ? n : f0->n_cells], beam, slack,
                                  cells, sc, &scored);
    if (ftau) {
        const int nt = ftau->prefix[n < ftau->n_cells ? n : ftau->n_cells];
        cnt += or_beam_forest(p, head, i, q_row, q_norm, ftau, nt, beam, slack, cells + cnt,
                              sc + cnt, &scored);
    }
    /* union of the two beams (a cell found twice has the same score) */
    or_beam_ent* u = (or_beam_ent*)malloc(sizeof(or_beam_ent) * (size_t)(cnt > 0 ? cnt : 1));
    int n_u = 0;
    for (int t = 0; t < cnt; ++t) {
        int dup = 0;
        for (int r = 0; r < n_u; ++r) dup |= u[r].first == cells[t];
        if (dup) continue;
        u[n_u].u = sc[t];
        u[n_u].first = cells[t];
        u[n_u].level = 0;
        u[n_u].index = 0;
        ++n_u;
    }
    qsort(u, (size_t)n_u, sizeof(or_beam_ent), or_cmp_beam);
    const int k = n_u < p->topk ? n_u : p->topk;
    for (int t = 0; t < k; ++t) {
        sel[t] = u[t].first;
        if (score) score[t] = u[t].u;
    }
    free(u);
    free(cells);
    free(sc);
    if (n_scored) *n_scored = scored;
    return k;
}
