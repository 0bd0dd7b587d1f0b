/*
 * fs.h -- C ABI of the FreeSolo FS-L sparse-attention forward on MI355X (gfx950).
 *
 * The operation is the FS-L forward of the FreeSolo paper summary (picx.dev page,
 * section 3 "Methodology"): per head, a RoPE sliding-window branch (section 3.2,
 * eqs. 3-4) plus a NoPE long-range branch over 32-token cells (section 3.3,
 * eqs. 5, 7, 8, 9), combined by eq. 2.  One entry point per step:
 *
 *   fs_cell_summaries  eq. 5   mean key and maximum token-key norm per cell
 *   fs_prune_prefix    eq. 8   FS-L query-independent pruning to W + P cells
 *                               (+ fs_prune_workspace_size)
 *   fs_select_topk     eq. 7   score q.kbar/sqrt(d) (+ optional erf prior), top-K cells
 *   fs_window_attn     eqs.3-4 RoPE attention over positions max(0,i-w) .. i
 *                               (+ fs_window_table / fs_window_attn_tabled)
 *   fs_sparse_attn     eq. 9   NoPE attention over the selected cells' tokens, RMSNorm
 *   fs_rerank_topk     eq. 12  token-level reranking (log-sum-exp of a cell's logits), top-K
 *   fs_stream_*        eqs. 2-9 from a bounded per-head state ("Bounded memory",
 *                      Practical Implications): decode or chunked prefill
 *   fs_combine         eq. 2   o = o_sr + alpha_h * o_lr
 *   fs_sparse_attn_combine  eqs. 9 + 2  the readout with eq. 2 in its epilogue
 *   fs_forest_*, fs_beam_select  eqs. 10-11  FS-B: causal forests over the cell
 *                      summaries and beam search for S_i (section 3.4)
 *
 * Readings of what the page leaves open (fixed here, identical in the oracle):
 *   - candidates of the query at position i are the complete cells whose last
 *     token precedes i - w: cells c < n_i = floor((i - w) / s) (0 when i < w);
 *   - the window holds the w + 1 positions max(0, i - w) .. i;
 *   - eq. 7's position prior is optional (absent = lambda_h 0); top-K and top-P
 *     ties go to the larger cell;
 *   - RoPE turns interleaved pairs (2k, 2k+1) by angle p * base^(-2k/d);
 *   - NoPE logits are q.k/sqrt(d); RMSNorm has unit gain; no selected cell gives 0.
 *
 * Conventions for every call:
 *   - All pointers except `problem` are DEVICE pointers, 16-byte aligned, owned
 *     by the caller.  The library allocates nothing and keeps no state between
 *     calls; calls are reentrant.  (The one exception is fs_sparse_attn_noalloc,
 *     whose scratch is a fixed device array of the library, one per GPU.)
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work; results are valid in stream order.
 *   - q, k, v, o_sr, o_lr and o hold elements of `problem->dtype`, addressed as
 *     base + b*stride[0] + h*stride[1] + t*stride[2] + e (element units, the d
 *     elements of a row contiguous).  Row strides must keep rows 16-byte aligned.
 *   - The other arrays are dense row-major with the shapes given per call.
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     FS_ERR_INVALID / FS_ERR_UNSUPPORTED is returned and nothing runs.  A failed
 *     launch returns FS_ERR_HIP.  A fault inside a kernel surfaces at the caller's
 *     next synchronisation.  fs_last_error() describes the last failure of the
 *     calling thread.  No exception or abort crosses this interface.
 */
#ifndef FS_H
#define FS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FS_OK = 0, FS_ERR_INVALID = 1, FS_ERR_UNSUPPORTED = 2, FS_ERR_HIP = 3 } fs_status;
typedef enum { FS_F32 = 0, FS_BF16 = 1 } fs_dtype;

typedef struct {
    int32_t batch, heads;     /* B, H >= 1 */
    int32_t head_dim;         /* d: 64 or 128 */
    int32_t n_ctx;            /* N: k and v hold positions 0 .. N-1 */
    int32_t n_q, q_pos0;      /* queries are positions q_pos0 .. q_pos0+n_q-1 <= N-1 */
    int32_t cell;             /* s: 32 */
    int32_t window;           /* w >= 0 */
    int32_t dtype;            /* fs_dtype of q, k, v, o_sr, o_lr, o */
    int32_t reserved;         /* 0 */
    int64_t q_stride[3];      /* (b, h, t) strides of q, in elements */
    int64_t kv_stride[3];     /* (b, h, t) strides of k and v */
    int64_t o_stride[3];      /* (b, h, t) strides of o_sr, o_lr and o */
} fs_problem;

/* Cell summaries, eq. 5.  For every complete cell c < C = floor(N / s):
 *   kbar[b][h][c][:] = mean of the raw (unrotated) keys of tokens cs .. cs+s-1
 *   amax[b][h][c]    = max over those tokens of ||k_j||_2
 * kbar: float32 [B][H][C][d]; amax: float32 [B][H][C].  The partial tail cell is
 * not summarised. */
fs_status fs_cell_summaries(const fs_problem* problem, const void* k, float* kbar, float* amax,
                            void* stream);

/* Host helper: the candidate counts the query block spans.  Query i has n_i
 * candidate cells; n_i is non-decreasing in i, so the block spans
 * n_lo = n_{q_pos0} .. n_lo + n_rows - 1 (n_rows = 0 when n_q = 0). */
fs_status fs_prune_rows(const fs_problem* problem, int32_t* n_lo, int32_t* n_rows);

/* FS-L prefix pruning, eq. 8.  Eq. 8's retained set depends on the query only
 * through n_i, so one row is written per candidate count n = n_lo + r:
 *   keep[b][h][r][0 .. cnt-1] = Recent_W({c < n}) U TopP_{c < n}(amax), ascending,
 *   keep[b][h][r][cnt ..]     = -1,       keep_count[b][h][r] = cnt <= W + P.
 * TopP orders by (amax, c) descending.  keep: int32 [B][H][n_rows][n_recent+budget];
 * keep_count: int32 [B][H][n_rows].  n_recent >= 0, budget >= 0,
 * 1 <= n_recent + budget <= 4096.  workspace (nullable, device, overwritten):
 * with at least fs_prune_workspace_size bytes, a call with many rows (a prefill)
 * finds each cell's eviction point once (the row count n from which P cells of
 * the prefix beat it) instead of searching every row; the rows are identical.
 * Calls sharing a workspace must not overlap in time. */
fs_status fs_prune_prefix(const fs_problem* problem, const float* amax, int32_t n_recent,
                          int32_t budget, int32_t* keep, int32_t* keep_count, void* workspace,
                          size_t ws_bytes, void* stream);

/* Bytes of the workspace fs_prune_prefix can use: one int32 per (b, h) and cell
 * below the largest candidate count the query block spans. */
fs_status fs_prune_workspace_size(const fs_problem* problem, size_t* bytes);

/* Scoring and top-K, eq. 7.  For each query i the score of cell c is
 * r_ic = q_i . kbar_c / sqrt(d) + lambda_h a_c erf((i - p_c) / (2 sigma_h)) with
 * the unrotated query and p_c = (c + 1/2) s (eq. 5).  The prior term is present
 * when prior_lambda is non-NULL; then amax ([B][H][C] as written by
 * fs_cell_summaries), prior_lambda and prior_sigma (float32 [H], lambda_h >= 0,
 * sigma_h > 0, device memory, not checked) are all required.  Candidates
 * are the keep row of n_i (keep != NULL; rows as written by fs_prune_prefix,
 * keep_width wide) or every cell c < n_i (keep == NULL: no pruning).  The
 * selected set is the min(topk, #candidates) candidates with the largest
 * (r_ic, c); it is written ascending to idx[b][h][t][:], padded with -1.
 * score (nullable) receives r_ic aligned with idx (0 for padding).
 * idx: int32 [B][H][n_q][topk]; score: float32 [B][H][n_q][topk]; 1 <= topk <= 64. */
fs_status fs_select_topk(const fs_problem* problem, const void* q, const float* kbar,
                         const float* amax, const float* prior_lambda, const float* prior_sigma,
                         const int32_t* keep, const int32_t* keep_count, int32_t keep_width,
                         int32_t topk, int32_t* idx, float* score, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of the optional workspace of fs_select_topk (keep_width 0: no pruning):
 * 0 unless the query range is short (fewer than 256 workgroups of 64 queries)
 * and the candidate union wider than 64 cells; then B H n_q S topk
 * (int32 cell + float32 key), S = ceil(union / 64) splits.  With such a
 * workspace (device memory, 256-byte aligned, owned by the caller) the union is
 * split over S workgroups per query tile, each ranking its 64 cells, and a merge
 * ranks their top-K lists again by the same keys; without one (NULL or smaller)
 * a single workgroup ranks the whole union.  The result does not depend on it.
 * Calls sharing one workspace on different streams race. */
fs_status fs_select_workspace_size(const fs_problem* problem, int32_t keep_width, int32_t topk,
                                   size_t* bytes);

/* Token-level reranking and top-K, eq. 12 (section 3.4): the same candidates,
 * prior and selection rule as fs_select_topk, with the score of cell c
 * r~_ic = log sum_{j in I_c} exp(q_i . k_j / sqrt(d)) + lambda_h a_c erf((i - p_c) / (2 sigma_h))
 * over the cell's s raw (unrotated) keys instead of the mean key.  k: [B][H][N][d]
 * with the problem's kv strides.  The prior arrays follow fs_select_topk's rule
 * (all NULL: no prior).  score (nullable) receives r~_ic aligned with idx.
 * workspace (nullable, device memory, 256-byte aligned, owned by the caller, not
 * kept after the call's work is done) of workspace_bytes >=
 * fs_rerank_workspace_size(problem, keep ? keep_width : 0) lets bf16 problems
 * score 128 queries per workgroup with the scores held there; a smaller or NULL
 * workspace uses a 64-query kernel that needs none.  The result does not depend
 * on it.  The 128-query kernel halves the workgroups: pass a workspace when
 * ceil(n_q / 128) B H is at least the device's compute-unit count, none for
 * short query ranges.  Calls sharing one workspace on different streams race. */
fs_status fs_rerank_topk(const fs_problem* problem, const void* q, const void* k,
                         const float* amax, const float* prior_lambda, const float* prior_sigma,
                         const int32_t* keep, const int32_t* keep_count, int32_t keep_width,
                         int32_t topk, int32_t* idx, float* score, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Bytes of the workspace fs_rerank_topk uses (keep_width 0: no pruning):
 * ceil(n_q / 128) B H round16(u) 128 float32 scores, u the most union cells of
 * the five candidate counts 128 queries span (keep_width + 5, or every candidate
 * cell without pruning). */
fs_status fs_rerank_workspace_size(const fs_problem* problem, int32_t keep_width,
                                   size_t* bytes);

/* ---- FS-B, section 3.4 (eqs. 10-11) -------------------------------------------
 * The page gives the admitted sets (eq. 10) and the node score (eq. 11) only;
 * the readings fixed here (identical in the oracle):
 *   - a causal forest over a sequence of cells is the set of complete, aligned
 *     power-of-two blocks: node (l, j) covers leaves j 2^l .. (j+1) 2^l - 1 and
 *     has children (l-1, 2j), (l-1, 2j+1); a prefix of n leaves is covered by
 *     one root per set bit of n.  Forest 0 holds every complete cell (A^0); a
 *     forest built with tau holds the cells with amax >= tau_h, ascending (A^tau).
 *     Query i searches the part of each forest that lies in C_i (cells < n_i);
 *   - mu_v = mean of the node's cell means, rho_v = the largest distance from
 *     mu_v to one of them, A_v = the largest amax, p_v^min = centre of the first
 *     cell.  With slack 1 and lambda_h >= 0, U_v bounds eq. 7's score of every
 *     cell below v;
 *   - beam search of width `beam` per forest: start from the best `beam` roots;
 *     each step replaces every inner node by its two children, keeps leaves and
 *     retains the best `beam` by U; stop when only leaves remain.  S_i is the
 *     best min(topk, #found) cells of both final beams by eq. 7's score (a
 *     leaf's U), written ascending like fs_select_topk.  Ties: larger U, then the
 *     later block (larger cell), then the lower level;
 *   - with token-level reranking (eq. 12, which the page places in FS-B), the
 *     found cells are ranked instead by r~ = log sum_j exp(q.k_j / sqrt(d)) over
 *     the cell's raw keys plus the same prior, ties to the larger cell; r~ is
 *     an fp32 dot product per key and an fp32 log-sum-exp.
 * U is computed in fp64 from the fp32 node statistics in one fixed order (dot
 * products as 16 contiguous partial sums added pairwise at distances 8, 4, 2,
 * 1), so the search's decisions are reproducible.
 *
 * Forest storage: fs_forest_size bytes of device memory (256-byte aligned, owned
 * by the caller) per forest, covering every (b, h); its layout is private to the
 * library.  A forest depends on batch, heads, head_dim and n_ctx only, so one
 * build serves any query range over the same cells.  The three calls accept at
 * most 32768 cells. */
fs_status fs_forest_size(const fs_problem* problem, size_t* bytes);

/* Builds one forest per (b, h) from kbar [B][H][C][d] and amax [B][H][C] (float32,
 * as written by fs_cell_summaries).  tau: NULL for forest 0 (every cell), or
 * float32 [H] thresholds for the admitted forest (amax >= tau_h).  Writes
 * `forest` only. */
fs_status fs_forest_build(const fs_problem* problem, const float* kbar, const float* amax,
                          const float* tau, void* forest, void* stream);

/* S_i by beam search (eq. 11) in forest0 and/or forest_tau (either may be NULL,
 * not both; each built with this problem's batch, heads, head_dim and n_ctx).
 * k: NULL to rank the found cells by eq. 7's score, or the raw keys [B][H][n_ctx][d]
 * (kv_stride, 16-byte aligned) to rank them by eq. 12's token-level score.
 * beam in [1, 64], slack c >= 0 (finite), topk in [1, 64].  prior_lambda,
 * prior_sigma: both NULL (no prior) or float32 [H] (lambda_h >= 0, sigma_h > 0,
 * not checked).  idx: int32 [B][H][n_q][topk], ascending, -1 padded; score
 * (nullable): float32, the ranking's score (eq. 7's, or eq. 12's with k) aligned
 * with idx (0 for padding); effort (nullable): int32 [B][H][n_q], the number of
 * node scores U_v the query's searches computed (its search effort: the node rows
 * it read). */
fs_status fs_beam_select(const fs_problem* problem, const void* q, const void* k,
                         const void* forest0, const void* forest_tau, int32_t beam, float slack,
                         const float* prior_lambda, const float* prior_sigma, int32_t topk,
                         int32_t* idx, float* score, int32_t* effort, void* stream);

/* Bytes of device workspace for fs_window_attn: its RoPE cos/sin table, then room
 * for the partial states with which a short query range (decode) splits each
 * query tile's keys over several workgroups. */
fs_status fs_workspace_size(const fs_problem* problem, size_t* bytes);

/* Local branch, eqs. 3-4: o_sr_i = softmax_j((R(i)q_i).(R(j)k_j)/sqrt(d)) v_j over
 * j = max(0, i-w) .. i, with RoPE base `rope_base`.  The kernel uses relative
 * angles, which eq. 3's right-hand side makes exact, so positions up to 2^31
 * lose no accuracy.  workspace (overwritten): at least the table; with
 * fs_workspace_size bytes a short query range splits its keys over workgroups.
 * Calls sharing a workspace must not overlap in time. */
fs_status fs_window_attn(const fs_problem* problem, const void* q, const void* k, const void* v,
                         float rope_base, void* workspace, size_t ws_bytes, void* o_sr,
                         void* stream);

/* The RoPE table of fs_window_attn's workspace alone (eq. 3's rotations by the
 * relative offsets -w-128 .. 127, cos/sin built in fp64, stored fp32).  It depends
 * only on the problem's window and head_dim and on rope_base, so a caller that
 * makes many window calls with the same three builds it once and then calls
 * fs_window_attn_tabled.  workspace: at least the table's bytes (the start of
 * fs_workspace_size). */
fs_status fs_window_table(const fs_problem* problem, float rope_base, void* workspace,
                          size_t ws_bytes, void* stream);

/* fs_window_attn without rebuilding the table: the workspace must already hold
 * the table that fs_window_table (or fs_window_attn) built for the same window,
 * head_dim and rope_base; it is read, not written (the split states after it are
 * overwritten).  A table built for other values is not detected and gives wrong
 * outputs. */
fs_status fs_window_attn_tabled(const fs_problem* problem, const void* q, const void* k,
                                const void* v, void* workspace, size_t ws_bytes, void* o_sr,
                                void* stream);

/* Bytes of device workspace with which fs_sparse_attn splits each query's cells
 * over several workgroups (0 when the query range already fills the device). */
fs_status fs_sparse_workspace_size(const fs_problem* problem, size_t* bytes);

/* Long-range readout, eq. 9: u_i = softmax_j(q_i.k_j/sqrt(d)) v_j over the tokens
 * of the cells listed in idx[b][h][t][0 .. topk-1] (-1 entries ignored; cells
 * must be < C and distinct), unrotated; o_lr_i = u_i / sqrt(mean(u_i^2) + rms_eps).
 * A query with no selected cell gets o_lr = 0.
 * workspace (nullable, device, overwritten): with at least
 * fs_sparse_workspace_size bytes, a short query range (decode) has its cells split
 * over workgroups whose partial softmax states are then merged; NULL runs
 * unsplit.  A non-NULL workspace below that size is an error.  Calls sharing a
 * workspace must not overlap in time. */
fs_status fs_sparse_attn(const fs_problem* problem, const void* q, const void* k, const void* v,
                         const int32_t* idx, int32_t topk, float rms_eps, void* workspace,
                         size_t ws_bytes, void* o_lr, void* stream);

/* fs_sparse_attn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * readout as fs_sparse_attn with a workspace of fs_sparse_workspace_size bytes,
 * with the split states held in a device array the library owns (16.25 MiB per
 * GPU, kept until the process ends) instead of a caller workspace.  It calls no
 * allocating routine.  The readout splits into at most 256 workgroups of 128
 * query rows, so no shape's states exceed the array (the 256k decode shape,
 * 8 heads x 256 queries x 16 splits x 520 bytes, fills it); a shape whose
 * states did would return FS_ERR_UNSUPPORTED and run nothing.  Every call on one GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must not be issued; the array keeps the last call's
 * states, which the next call overwrites before reading. */
fs_status fs_sparse_attn_noalloc(const fs_problem* problem, const void* q, const void* k,
                                 const void* v, const int32_t* idx, int32_t topk, float rms_eps,
                                 void* o_lr, void* stream);

/* The long-range readout (eq. 9, as fs_sparse_attn) with the range combination
 * (eq. 2) in its epilogue: o = o_sr + alpha[h] * o_lr, o_lr kept in fp32 until
 * the sum (fs_sparse_attn followed by fs_combine rounds it to the storage type
 * first, so bf16 results may differ by one rounding of alpha_h o_lr).  o_sr and
 * o: [B][H][n_q][d] with the problem's o_stride; o may be o_sr itself (each
 * element is read before it is written, by the same thread).  alpha: float32
 * [H].  workspace / ws_bytes as for fs_sparse_attn.  One fewer pass over the
 * branch outputs than the two calls. */
fs_status fs_sparse_attn_combine(const fs_problem* problem, const void* q, const void* k,
                                 const void* v, const int32_t* idx, int32_t topk, float rms_eps,
                                 const void* o_sr, const float* alpha, void* workspace,
                                 size_t ws_bytes, void* o, void* stream);

/* Range combination, eq. 2: o = o_sr + alpha[h] * o_lr.  alpha: float32 [H]. */
fs_status fs_combine(const fs_problem* problem, const void* o_sr, const void* o_lr,
                     const float* alpha, void* o, void* stream);

/* ---- Streaming FS-L: eqs. 2-9 from a fixed-size per-head state ---------------
 * The page's bounded-memory claim (Practical Implications, "Bounded memory"): FS-L
 * needs O((P + W) s + w + B + s) d token state per head, independent of the
 * sequence length, because eq. 8 discards a cell for good once it leaves both
 * Recent_W and TopP (TopP over a longer prefix only ever takes the new cell).
 * The state, one opaque device buffer owned by the caller, holds per (b, h): the
 * last L >= w + s + max_new raw keys/values, the retained cells' raw keys/values
 * and summaries in W + P + ceil(max_new / s) + 2 slots, and eq. 8's sets.  Its
 * size depends on the config only, never on how many tokens have been appended. */
typedef struct {
    int32_t batch, heads, head_dim;   /* B, H, d (64 or 128) */
    int32_t cell, window;             /* s (32), w (>= 0) */
    int32_t n_recent, budget;         /* W, P of eq. 8: W, P >= 0, 1 <= W + P <= 1024 */
    int32_t topk;                     /* K of eq. 9's selection, 1 .. 64 */
    int32_t max_new;                  /* most tokens one step appends, 1 .. 4096 */
    fs_dtype dtype;                   /* storage dtype of q/k/v/o and of the state */
    float rope_base;                  /* RoPE base of eq. 3 (> 1) */
    float rms_eps;                    /* RMSNorm epsilon of eq. 9 (>= 0) */
} fs_stream_config;

/* Bytes of the state buffer for a config. */
fs_status fs_stream_state_size(const fs_stream_config* cfg, size_t* bytes);

/* Empty the state (no tokens) and tabulate the window's rotations.  state: device,
 * 256-byte aligned, >= the size above. */
fs_status fs_stream_reset(const fs_stream_config* cfg, void* state, size_t state_bytes,
                          void* stream);

/* One step: append the tokens at positions pos0 .. pos0 + n_new - 1 (k, v) of every
 * (b, h) and return, for the queries q at those same positions, the FS-L output of
 * eq. 2 (o_sr of eqs. 3-4 + alpha_h o_lr of eqs. 5, 7, 8, 9), computed from the state
 * alone.  Equal to the fs_* calls above on the whole prefix for those queries.
 * pos0 must be the number of tokens appended since the reset (not checked on the
 * device), pos0 + n_new < 2^31, 1 <= n_new <= max_new.  q, k, v, o: contiguous
 * [B][H][n_new][d] in the config's dtype (device, 16-byte aligned).  alpha: float32
 * [H].  prior_lambda, prior_sigma: both NULL (no prior) or both float32 [H] (eq. 7).
 * idx (nullable): int32 [B][H][n_new][topk], the selected cells (absolute cell
 * indices, ascending, -1 padded).  Steps on one state must not overlap in time. */
fs_status fs_stream_step(const fs_stream_config* cfg, void* state, size_t state_bytes,
                         int64_t pos0, int32_t n_new, const void* q, const void* k,
                         const void* v, const float* alpha, const float* prior_lambda,
                         const float* prior_sigma, void* o, int32_t* idx, void* stream);

const char* fs_status_string(fs_status status);
const char* fs_last_error(void);

/* The kernel path the calling thread's last readout, window, selection or
 * reranking call chose: the MFMA kernels (and their split count), or a row-wise
 * fallback and its reason (fp32 storage, a union wider than the MFMA kernels'
 * register blocks, too little LDS, too many cells).  Empty before any such
 * call; valid until the thread's next call. */
const char* fs_last_path(void);

#ifdef __cplusplus
}
#endif
#endif /* FS_H */
