/*
 * fs_oracle.h -- plain fp64 CPU oracle of the FreeSolo FS-L attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path (the
 * HIP library and its Python binding) never calls it and shares no code,
 * header, table or helper with it.
 *
 * Source: the FreeSolo paper summary (picx.dev page), section "Methodology",
 * eqs. (2)-(5) and (7)-(9).  Every function says which equation it follows.
 * Readings of what the page leaves open:
 *   - candidate cells of query i are the complete cells whose last token is
 *     before i - w (the definition of C_i, eq. 6, is missing from the page);
 *   - the window of eq. (4) holds the w + 1 positions max(0, i - w) .. i;
 *   - eq. (7)'s position prior lambda_h a_c erf((i - p_c) / (2 sigma_h)) is on
 *     when the problem carries per-head lambda and sigma arrays, else 0;
 *   - RoPE rotates interleaved pairs (2k, 2k+1) by angle p * base^(-2k/d);
 *   - ties in TopP and top-K go to the larger cell index;
 *   - the NoPE logits of eq. (9) are q.k / sqrt(d); RMSNorm has unit gain and
 *     the epsilon given in the problem; an empty selection gives o_lr = 0.
 *
 * Layout: q is [B, H, n_q, d], k and v are [B, H, N, d], row-major float32
 * holding the exact stored values (bf16 inputs are widened without rounding).
 * All arithmetic is in double.
 */
#ifndef FS_ORACLE_H
#define FS_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int batch, heads, head_dim, n_ctx;
    int n_q, q_pos0;          /* queries are positions q_pos0 .. q_pos0 + n_q - 1 */
    int cell, window;         /* s and w */
    int topk;                 /* K */
    int budget;               /* P; negative means no pruning (A_i = C_i) */
    int n_recent;             /* W */
    double rope_base;
    double rms_eps;
    long long pos_offset;     /* absolute position of token 0; RoPE angles only */
    /* eq. (7) prior, per head: lambda_h >= 0, sigma_h > 0 (both NULL: no prior) */
    const double* prior_lambda;
    const double* prior_sigma;
} or_problem;

/* Position prior of eq. (7) for the query at position i and cell c of head h:
 * lambda_h a_c erf((i - p_c) / (2 sigma_h)) with p_c = (c + 1/2) s (eq. 5);
 * 0 without prior arrays.  Positions are token indices; only i - p_c enters. */
double or_prior(const or_problem* p, int head, long long i, int c, double a_c);

/* RoPE rotation R(pos) of one d-vector (eq. 3). */
void or_rope(const or_problem* p, const float* x, long long pos, double* out);

/* Number of candidate cells n_i of the query at position i (C_i = {c < n_i}). */
int or_n_candidates(const or_problem* p, long long i);

/* Cell summaries of one head (eq. 5): kbar [C, d] and amax [C], C = N / s. */
void or_cell_summaries_head(const or_problem* p, const float* k_head, double* kbar, double* amax);

/* FS-L pruning (eq. 8) of the candidate set {c < n}: writes the retained cells in
 * ascending order to keep and returns their number.  gap_rel (nullable) receives
 * the relative gap between the P-th and (P+1)-th priorities, or +inf. */
int or_prune_row(const or_problem* p, const double* amax, int n, int* keep, double* gap_rel);

/* Cell scores r_c = q.kbar_c / sqrt(d) + or_prior(p, head, i, c, amax[c]) (eq. 7)
 * over cand, and the top-min(K, n_cand) cells written ascending to sel; returns
 * their number.  amax may be NULL when the problem has no prior.
 * gap_rel (nullable): relative gap between the K-th and (K+1)-th scores, or +inf.
 * cand_scores (nullable): the score of every candidate, in cand order. */
int or_select_row_at(const or_problem* p, int head, long long i, const float* q_row,
                     const double* kbar, const double* amax, const int* cand, int n_cand,
                     int* sel, double* gap_rel, double* cand_scores);

/* Token-level reranking (eq. 12): r~_c = log sum_{j in I_c} exp(q.k_j / sqrt(d))
 * + or_prior(p, head, i, c, amax[c]) over cand, with the unrotated query and the
 * cell's s raw keys; then the same top-K as or_select_row_at. */
int or_rerank_row(const or_problem* p, int head, long long i, const float* q_row,
                  const float* k_head, const double* amax, const int* cand, int n_cand,
                  int* sel, double* gap_rel, double* cand_scores);

/* or_select_row_at without the prior (content score only). */
int or_select_row(const or_problem* p, const float* q_row, const double* kbar,
                  const int* cand, int n_cand, int* sel, double* gap_rel, double* cand_scores);

/* Local branch (eqs. 3-4) of the query at position i. */
void or_window_row(const or_problem* p, const float* q_row, const float* k_head,
                   const float* v_head, long long i, double* o_sr);

/* Long-range readout (eq. 9) over the tokens of the n_sel cells in sel. */
void or_sparse_row(const or_problem* p, const float* q_row, const float* k_head,
                   const float* v_head, const int* sel, int n_sel, double* o_lr);

/* Whole forward of head `head` for a list of query rows t (0 <= t < n_q), threaded.
 * kbar/amax: summaries of this head.  keep_ovr/sel_ovr (nullable) replace the
 * retained / selected sets of a row when the row's count in *_ovr_n is >= 0;
 * rows are keep_w / topk ints wide.  Outputs per row: o, o_sr, o_lr [d];
 * sel [topk] (-1 padded) with its count n_sel; the two boundary gaps. */
int or_forward_rows(const or_problem* p, const float* q_head, const float* k_head,
                    const float* v_head, const double* kbar, const double* amax,
                    double alpha, const int* rows, int n_rows,
                    const int* keep_ovr, const int* keep_ovr_n, int keep_w,
                    const int* sel_ovr, const int* sel_ovr_n,
                    double* o, double* o_sr, double* o_lr, int* sel, int* n_sel,
                    double* sel_gap, double* keep_gap, int nthreads, int head);

/* Whole forward of the whole problem (eq. 2 for every b, h, query), threaded. */
int or_forward(const or_problem* p, const float* q, const float* k, const float* v,
               const float* alpha, double* o, double* o_sr, double* o_lr,
               int* sel, int* n_sel, double* sel_gap, double* keep_gap, int nthreads);


/* ---- FS-B: causal forests and beam search (section 3.4, eqs. 10-11) ------
 * Readings and the decision precision are stated in fsb_oracle.c.  A forest
 * is built over one head's fp32 cell summaries; the caller allocates every
 * array: cell_of [C], prefix [C + 1], first / amax / rho [2C], mu [2C * d]. */
typedef struct {
    int n_cells, head_dim;
    int m;                 /* admitted cells (leaves) */
    int n_levels;          /* levels 0 .. n_levels - 1 */
    int level_start[32];   /* node (l, j) is node level_start[l] + j */
    int* cell_of;          /* leaf j -> cell, ascending */
    int* prefix;           /* prefix[n] = admitted cells among cells 0 .. n-1 */
    int* first;            /* node -> its first cell */
    float* amax;           /* node -> A_v */
    float* rho;            /* node -> rho_v */
    float* mu;             /* node -> mu_v [d] */
} or_forest;

/* Dot product of two d-vectors (d a multiple of 16) in the fixed fp64 order. */
double or_dot16(const float* a, const float* b, int d);

/* Builds the forest of the cells with amax >= tau (use_tau), or of every cell;
 * returns the number of leaves. */
int or_forest_build(const float* kbar, const float* amax, int n_cells, int d, int use_tau,
                    double tau, or_forest* f);

/* Roots (level, index) covering the first n_leaves leaves, largest first. */
int or_forest_roots(const or_forest* f, int n_leaves, int* level, int* index);

/* U_v of node (level, index) for the query at position i of head `head` (eq. 11);
 * q_norm = sqrt(or_dot16(q, q)). */
double or_node_score(const or_problem* p, int head, long long i, const float* q_row,
                     double q_norm, const or_forest* f, int level, int index, double slack);

/* S_i of the query at position i: beam search of width `beam` in f0 and ftau
 * (either may be NULL), then the best min(K, |found|) by eq. 7's score, in
 * descending (score, cell) order.  Returns the count; *n_scored (nullable)
 * receives the number of node scores U_v the two searches computed. */
int or_beam_row(const or_problem* p, int head, long long i, const float* q_row,
                const or_forest* f0, const or_forest* ftau, int beam, double slack,
                int* sel, double* score, int* n_scored);

/* ---- FS-B in plain fp64 (fsb_plain.c) -------------------------------------
 * The same readings, with fp64 node statistics from fp64 cell summaries and
 * dot products in index order.  The caller allocates cell_of [C], prefix
 * [C + 1], first [2C], amax / rho [2C], mu [2C * d]. */
typedef struct {
    int n_cells, head_dim;
    int m;
    int n_levels;
    int level_start[32];
    int* cell_of;
    int* prefix;
    int* first;
    double* amax;
    double* rho;
    double* mu;
} or_forest64;

int or_forest64_build(const double* kbar, const double* amax, int n_cells, int d, int use_tau,
                      double tau, or_forest64* f);

/* Roots (level, index) covering the first n leaves, largest first. */
int or_forest64_roots(const or_forest64* f, int n, int* level, int* index);

double or_node64_score(const or_problem* p, int head, long long i, const float* q_row,
                       const or_forest64* f, int level, int index, double slack);

/* S_i of one query (as or_beam_row); *gap (nullable) receives the smallest
 * relative gap of the search's cuts and of the final top-K (+inf: none). */
int or_beam64_row(const or_problem* p, int head, long long i, const float* q_row,
                  const or_forest64* f0, const or_forest64* ftau, int beam, double slack,
                  int* sel, double* score, int* n_scored, double* gap);

/* The cells both searches of or_beam64_row end with, without repeats (at most
 * 2 beam), in search order; *gap receives the smallest relative gap of the
 * searches' cuts.  Eq. 12's reranking over them is or_rerank_row with these
 * cells as candidates. */
int or_beam64_found(const or_problem* p, int head, long long i, const float* q_row,
                    const or_forest64* f0, const or_forest64* ftau, int beam, double slack,
                    int* cells, int* n_scored, double* gap);

/* or_beam64_row for the query rows t in `rows` (positions q_pos0 + t) of head
 * `head`, threaded.  Per row: sel / score [topk] in descending (score, cell)
 * order, -1 / 0 padded; n_sel; n_scored; gap. */
int or_beam64_rows(const or_problem* p, int head, const float* q_head, const int* rows,
                   int n_rows, const or_forest64* f0, const or_forest64* ftau, int beam,
                   double slack, int* sel, double* score, int* n_sel, int* n_scored,
                   double* gap, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
