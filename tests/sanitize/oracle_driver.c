/*
 * oracle_driver.c -- runs every entry point of the CPU oracle (oracle/*.c) on
 * small seeded problems, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize_cpu.py builds and runs it).
 * Test infrastructure: it checks memory and UB safety of the oracle, not its
 * values (the pins do that).
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fs_oracle.h"

static unsigned long long g_state = 88172645463325252ull;
static float rnd(void)   /* xorshift64, uniform in [-1, 1) */
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (float)((double)(g_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static float* fill(size_t n)
{
    float* x = (float*)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) x[i] = rnd();
    return x;
}

static int run(int n_ctx, int d, int window, int topk, int budget, int n_recent, int with_prior)
{
    or_problem p;
    memset(&p, 0, sizeof(p));
    p.batch = 1; p.heads = 2; p.head_dim = d; p.n_ctx = n_ctx; p.n_q = n_ctx; p.q_pos0 = 0;
    p.cell = 32; p.window = window; p.topk = topk; p.budget = budget; p.n_recent = n_recent;
    p.rope_base = 10000.0; p.rms_eps = 1e-6; p.pos_offset = 0;
    double lam[2] = {0.1, 0.2}, sig[2] = {300.0, 900.0};
    if (with_prior) { p.prior_lambda = lam; p.prior_sigma = sig; }
    const int H = p.heads, C = n_ctx / 32;
    const size_t nh = (size_t)n_ctx * d;
    float *q = fill(H * nh), *k = fill(H * nh), *v = fill(H * nh);
    float alpha[2] = {0.5f, 0.25f};
    double* kbar = (double*)malloc(sizeof(double) * (size_t)(C ? C : 1) * d);
    double* amax = (double*)malloc(sizeof(double) * (C ? C : 1));
    or_cell_summaries_head(&p, k, kbar, amax);

    double rot[128];
    or_rope(&p, q, 12345, rot);
    int* keep = (int*)malloc(sizeof(int) * (size_t)(C + 1));
    int* cand = (int*)malloc(sizeof(int) * (size_t)(C + 1));
    int* sel = (int*)malloc(sizeof(int) * (size_t)(C + 1));
    double* scores = (double*)malloc(sizeof(double) * (size_t)(C + 1));
    double out[128], gap;
    for (int i = 0; i < n_ctx; i += 37) {
        const int n = or_n_candidates(&p, i);
        int cnt = n;
        if (budget >= 0) cnt = or_prune_row(&p, amax, n, keep, &gap);
        for (int t = 0; t < cnt; ++t) cand[t] = budget >= 0 ? keep[t] : t;
        const int ns = or_select_row_at(&p, 1, i, q + nh + (size_t)i * d, kbar, amax, cand, cnt,
                                        sel, &gap, scores);
        or_select_row(&p, q + (size_t)i * d, kbar, cand, cnt, sel, &gap, NULL);
        or_rerank_row(&p, 0, i, q + (size_t)i * d, k, amax, cand, cnt, sel, &gap, scores);
        or_window_row(&p, q + (size_t)i * d, k, v, i, out);
        or_sparse_row(&p, q + (size_t)i * d, k, v, sel, ns, out);
        (void)or_prior(&p, 1, i, 0, 1.0);
    }
    /* the threaded forward, with and without overrides */
    const int nr = n_ctx / 3 + 1;
    int* rows = (int*)malloc(sizeof(int) * nr);
    for (int r = 0; r < nr; ++r) rows[r] = (r * 3) % n_ctx;
    double *o = (double*)malloc(sizeof(double) * nr * d), *osr = (double*)malloc(sizeof(double) * nr * d);
    double* olr = (double*)malloc(sizeof(double) * nr * d);
    int* sl = (int*)malloc(sizeof(int) * nr * topk);
    int* nsel = (int*)malloc(sizeof(int) * nr);
    double *sg = (double*)malloc(sizeof(double) * nr), *kg = (double*)malloc(sizeof(double) * nr);
    or_forward_rows(&p, q, k, v, kbar, amax, 0.5, rows, nr, NULL, NULL, 0, NULL, NULL, o, osr,
                    olr, sl, nsel, sg, kg, 4, 0);
    int* ovr = (int*)malloc(sizeof(int) * nr * topk);
    int* ovr_n = (int*)malloc(sizeof(int) * nr);
    for (int r = 0; r < nr; ++r) {
        ovr_n[r] = r % 2 ? -1 : (C < topk ? C : topk) / 2;
        for (int t = 0; t < topk; ++t) ovr[r * topk + t] = t < ovr_n[r] ? t : -1;
    }
    or_forward_rows(&p, q, k, v, kbar, amax, 0.5, rows, nr, NULL, NULL, 0, ovr, ovr_n, o, osr,
                    olr, sl, nsel, sg, kg, 3, 1);
    double* ofull = (double*)malloc(sizeof(double) * H * nh);
    double* ofsr = (double*)malloc(sizeof(double) * H * nh);
    double* oflr = (double*)malloc(sizeof(double) * H * nh);
    int* fsel = (int*)malloc(sizeof(int) * (size_t)H * n_ctx * topk);
    int* fns = (int*)malloc(sizeof(int) * (size_t)H * n_ctx);
    double* fsg = (double*)malloc(sizeof(double) * (size_t)H * n_ctx);
    double* fkg = (double*)malloc(sizeof(double) * (size_t)H * n_ctx);
    or_forward(&p, q, k, v, alpha, ofull, ofsr, oflr, fsel, fns, fsg, fkg, 4);

    /* FS-B: both oracles, both forests */
    if (C > 0) {
        float* kb32 = (float*)malloc(sizeof(float) * (size_t)C * d);
        float* am32 = (float*)malloc(sizeof(float) * C);
        for (int c = 0; c < C; ++c) {
            am32[c] = (float)amax[c];
            for (int e = 0; e < d; ++e) kb32[(size_t)c * d + e] = (float)kbar[(size_t)c * d + e];
        }
        int lv[32], ix[32];
        or_forest f32s[2];
        or_forest64 f64s[2];
        for (int t = 0; t < 2; ++t) {
            or_forest* f = &f32s[t];
            memset(f, 0, sizeof(*f));
            f->cell_of = (int*)malloc(sizeof(int) * C); f->prefix = (int*)malloc(sizeof(int) * (C + 1));
            f->first = (int*)malloc(sizeof(int) * 2 * C); f->amax = (float*)malloc(sizeof(float) * 2 * C);
            f->rho = (float*)malloc(sizeof(float) * 2 * C); f->mu = (float*)malloc(sizeof(float) * 2 * (size_t)C * d);
            or_forest_build(kb32, am32, C, d, t, 0.9 * amax[0], f);
            or_forest64* g = &f64s[t];
            memset(g, 0, sizeof(*g));
            g->cell_of = (int*)malloc(sizeof(int) * C); g->prefix = (int*)malloc(sizeof(int) * (C + 1));
            g->first = (int*)malloc(sizeof(int) * 2 * C); g->amax = (double*)malloc(sizeof(double) * 2 * C);
            g->rho = (double*)malloc(sizeof(double) * 2 * C); g->mu = (double*)malloc(sizeof(double) * 2 * (size_t)C * d);
            or_forest64_build(kbar, amax, C, d, t, 0.9 * amax[0], g);
            or_forest_roots(f, C, lv, ix);
            or_forest64_roots(g, C, lv, ix);
        }
        int ns;
        for (int i = 0; i < n_ctx; i += 53) {
            or_beam_row(&p, 0, i, q + (size_t)i * d, &f32s[0], &f32s[1], 4, 1.0, sel, scores, &ns);
            or_beam64_row(&p, 0, i, q + (size_t)i * d, &f64s[0], &f64s[1], 4, 1.0, sel, scores,
                          &ns, &gap);
            /* eq. 12 over the found cells (at most 2 beam + 2 of them) */
            int found[10];
            const int nf = or_beam64_found(&p, 0, i, q + (size_t)i * d, &f64s[0], &f64s[1], 4,
                                           1.0, found, &ns, &gap);
            or_rerank_row(&p, 0, i, q + (size_t)i * d, k, amax, found, nf, sel, &gap, scores);
        }
        int* bsel = (int*)malloc(sizeof(int) * nr * topk);
        double* bsc = (double*)malloc(sizeof(double) * nr * topk);
        int *bn = (int*)malloc(sizeof(int) * nr), *be = (int*)malloc(sizeof(int) * nr);
        double* bg = (double*)malloc(sizeof(double) * nr);
        or_beam64_rows(&p, 1, q + nh, rows, nr, &f64s[0], NULL, 8, 0.5, bsel, bsc, bn, be, bg, 4);
        (void)or_dot16(kb32, kb32, d);
        free(bsel); free(bsc); free(bn); free(be); free(bg);
        for (int t = 0; t < 2; ++t) {
            free(f32s[t].cell_of); free(f32s[t].prefix); free(f32s[t].first); free(f32s[t].amax);
            free(f32s[t].rho); free(f32s[t].mu);
            free(f64s[t].cell_of); free(f64s[t].prefix); free(f64s[t].first); free(f64s[t].amax);
            free(f64s[t].rho); free(f64s[t].mu);
        }
        free(kb32); free(am32);
    }
    free(q); free(k); free(v); free(kbar); free(amax); free(keep); free(cand); free(sel);
    free(scores); free(rows); free(o); free(osr); free(olr); free(sl); free(nsel); free(sg);
    free(kg); free(ovr); free(ovr_n); free(ofull); free(ofsr); free(oflr); free(fsel); free(fns);
    free(fsg); free(fkg);
    return 0;
}

int main(void)
{
    /* shapes: unpruned and pruned, Recent_W, the prior, no complete cell, one cell,
       a window wider than the context, d 64 and 128 */
    run(700, 64, 512, 8, -1, 0, 0);
    run(1500, 128, 256, 5, 9, 3, 1);
    run(20, 64, 512, 4, 3, 0, 0);
    run(45, 64, 0, 2, 3, 0, 1);
    run(640, 64, 704, 8, 4, 0, 0);
    puts("oracle driver: done");
    return 0;
}
