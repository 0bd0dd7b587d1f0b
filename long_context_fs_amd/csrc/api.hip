// api.hip -- the C ABI of include/fs.h: host-side validation, launch, error mapping.
//
// Every entry point validates its arguments on the host and enqueues nothing on
// failure.  No exception or abort crosses the interface.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/fs.h"
#include "fs_launch.hpp"
#include "fs_stream.hpp"

namespace {

thread_local char g_err[512];
thread_local char g_path[256];

fs_status fail(fs_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

fs_status from_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) {
        g_err[0] = 0;
        return FS_OK;
    }
    return fail(FS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validate the problem and build the kernels' view of it.
fs_status check_problem(const fs_problem* p, fs::Shape* sh)
{
    if (!p) return fail(FS_ERR_INVALID, "problem is NULL");
    if (p->batch < 1 || p->heads < 1) return fail(FS_ERR_INVALID, "batch and heads must be >= 1");
    if ((long)p->batch * p->heads > 65535)
        return fail(FS_ERR_UNSUPPORTED, "batch * heads must be <= 65535");
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(FS_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128", p->head_dim);
    if (p->cell != 32) return fail(FS_ERR_UNSUPPORTED, "cell %d: only 32", p->cell);
    if (p->dtype != FS_F32 && p->dtype != FS_BF16)
        return fail(FS_ERR_INVALID, "dtype %d", p->dtype);
    if (p->n_ctx < 1) return fail(FS_ERR_INVALID, "n_ctx must be >= 1");
    if (p->window < 0 || p->window > (1 << 20))
        return fail(FS_ERR_UNSUPPORTED, "window %d outside [0, 2^20]", p->window);
    if (p->n_q < 0 || p->q_pos0 < 0 || (long)p->q_pos0 + p->n_q > p->n_ctx)
        return fail(FS_ERR_INVALID, "queries %d..%d outside 0..n_ctx-1 (%d)", p->q_pos0,
                    p->q_pos0 + p->n_q - 1, p->n_ctx);
    if (p->reserved != 0) return fail(FS_ERR_INVALID, "reserved field must be 0");
    const int epv = p->dtype == FS_BF16 ? 8 : 4;   // elements per 16 bytes
    const int64_t* strides[3] = {p->q_stride, p->kv_stride, p->o_stride};
    const char* names[3] = {"q_stride", "kv_stride", "o_stride"};
    for (int a = 0; a < 3; ++a) {
        for (int t = 0; t < 3; ++t) {
            if (strides[a][t] < 0 || strides[a][t] % epv != 0)
                return fail(FS_ERR_INVALID, "%s[%d] = %lld must be >= 0 and keep rows 16-byte aligned",
                            names[a], t, (long long)strides[a][t]);
        }
        if (strides[a][2] < p->head_dim)
            return fail(FS_ERR_INVALID, "%s[2] must be >= head_dim", names[a]);
    }
    sh->B = p->batch; sh->H = p->heads; sh->d = p->head_dim; sh->N = p->n_ctx;
    sh->nq = p->n_q; sh->q_pos0 = p->q_pos0; sh->s = p->cell; sh->w = p->window;
    sh->bf16 = p->dtype == FS_BF16;
    sh->C = p->n_ctx / p->cell;
    for (int t = 0; t < 3; ++t) {
        sh->qs[t] = p->q_stride[t];
        sh->kvs[t] = p->kv_stride[t];
        sh->os[t] = p->o_stride[t];
    }
    return FS_OK;
}

#define FS_CHECK(call)                    \
    do {                                  \
        fs_status st_ = (call);           \
        if (st_ != FS_OK) return st_;     \
    } while (0)

#define FS_PTR(ptr)                                                                      \
    do {                                                                                 \
        if (!(ptr)) return fail(FS_ERR_INVALID, "%s is NULL", #ptr);                     \
        if (!aligned16(ptr)) return fail(FS_ERR_INVALID, "%s is not 16-byte aligned", #ptr); \
    } while (0)

}  // namespace

namespace fs {
void note_path(const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_path, sizeof(g_path), fmt, ap);
    va_end(ap);
}
}  // namespace fs

namespace fs {
void candidate_rows(const Shape& sh, int* n_lo, int* n_rows)
{
    auto ncand = [&](long i) -> int {
        if (i < sh.w) return 0;
        long n = (i - sh.w) / sh.s;
        return (int)(n < sh.C ? n : sh.C);
    };
    if (sh.nq == 0) {
        *n_lo = 0;
        *n_rows = 0;
        return;
    }
    *n_lo = ncand(sh.q_pos0);
    *n_rows = ncand((long)sh.q_pos0 + sh.nq - 1) - *n_lo + 1;
}
}  // namespace fs

extern "C" {

const char* fs_status_string(fs_status s)
{
    switch (s) {
        case FS_OK: return "FS_OK";
        case FS_ERR_INVALID: return "FS_ERR_INVALID";
        case FS_ERR_UNSUPPORTED: return "FS_ERR_UNSUPPORTED";
        case FS_ERR_HIP: return "FS_ERR_HIP";
    }
    return "unknown fs_status";
}

const char* fs_last_error(void) { return g_err; }

const char* fs_last_path(void) { return g_path; }

fs_status fs_cell_summaries(const fs_problem* problem, const void* k, float* kbar, float* amax,
                            void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(k); FS_PTR(kbar);
    if (!amax) return fail(FS_ERR_INVALID, "amax is NULL");
    return from_hip(fs::launch_summaries(sh, k, kbar, amax, (hipStream_t)stream),
                    "fs_cell_summaries");
}

fs_status fs_prune_rows(const fs_problem* problem, int32_t* n_lo, int32_t* n_rows)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!n_lo || !n_rows) return fail(FS_ERR_INVALID, "n_lo / n_rows is NULL");
    int lo, rows;
    fs::candidate_rows(sh, &lo, &rows);
    *n_lo = lo;
    *n_rows = rows;
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_prune_workspace_size(const fs_problem* problem, size_t* bytes)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    *bytes = fs::prune_ws_bytes(sh);
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_prune_prefix(const fs_problem* problem, const float* amax, int32_t n_recent,
                          int32_t budget, int32_t* keep, int32_t* keep_count, void* workspace,
                          size_t ws_bytes, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (n_recent < 0 || budget < 0 || n_recent + budget < 1 || n_recent + budget > 4096)
        return fail(FS_ERR_UNSUPPORTED, "n_recent %d + budget %d must be in [1, 4096]", n_recent,
                    budget);
    if (!amax || !keep || !keep_count) return fail(FS_ERR_INVALID, "NULL amax/keep/keep_count");
    if (workspace && ws_bytes < fs::prune_ws_bytes(sh))
        return fail(FS_ERR_INVALID, "workspace of %zu bytes, need %zu", ws_bytes,
                    fs::prune_ws_bytes(sh));
    if (workspace && ((uintptr_t)workspace & 15))
        return fail(FS_ERR_INVALID, "workspace is not 16-byte aligned");
    int lo, rows;
    fs::candidate_rows(sh, &lo, &rows);
    return from_hip(fs::launch_prune(sh, amax, lo, rows, n_recent, budget, keep, keep_count,
                                     (hipStream_t)stream, workspace, ws_bytes),
                    "fs_prune_prefix");
}

fs_status fs_select_topk(const fs_problem* problem, const void* q, const float* kbar,
                         const float* amax, const float* prior_lambda, const float* prior_sigma,
                         const int32_t* keep, const int32_t* keep_count, int32_t keep_width,
                         int32_t topk, int32_t* idx, float* score, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(kbar);
    if (workspace && ((uintptr_t)workspace & 255))
        return fail(FS_ERR_INVALID, "workspace must be 256-byte aligned");
    if (prior_lambda && (!prior_sigma || !amax))
        return fail(FS_ERR_INVALID, "the position prior needs amax, prior_lambda and prior_sigma");
    if (!idx) return fail(FS_ERR_INVALID, "idx is NULL");
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    if (keep && (!keep_count || keep_width < 1 || keep_width > 4096))
        return fail(FS_ERR_INVALID, "keep needs keep_count and keep_width in [1, 4096]");
    int lo, rows;
    fs::candidate_rows(sh, &lo, &rows);
    if (!keep) {
        long last = (long)sh.q_pos0 + sh.nq - 1;
        long n_hi = last >= sh.w ? (last - sh.w) / sh.s : 0;
        if (n_hi > 16256)
            return fail(FS_ERR_UNSUPPORTED, "without pruning at most 16256 candidate cells");
    }
    const fs::Prior pr{amax, prior_lambda, prior_sigma};
    return from_hip(fs::launch_select(sh, q, kbar, pr, keep, keep_count, keep_width, lo, rows,
                                      topk, idx, score, workspace,
                                      workspace ? workspace_bytes : 0, (hipStream_t)stream),
                    "fs_select_topk");
}

fs_status fs_rerank_topk(const fs_problem* problem, const void* q, const void* k,
                         const float* amax, const float* prior_lambda, const float* prior_sigma,
                         const int32_t* keep, const int32_t* keep_count, int32_t keep_width,
                         int32_t topk, int32_t* idx, float* score, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(k);
    if (workspace && ((uintptr_t)workspace & 255))
        return fail(FS_ERR_INVALID, "workspace must be 256-byte aligned");
    if (prior_lambda && (!prior_sigma || !amax))
        return fail(FS_ERR_INVALID, "the position prior needs amax, prior_lambda and prior_sigma");
    if (!idx) return fail(FS_ERR_INVALID, "idx is NULL");
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    if (keep && (!keep_count || keep_width < 1 || keep_width > 4096))
        return fail(FS_ERR_INVALID, "keep needs keep_count and keep_width in [1, 4096]");
    int lo, rows;
    fs::candidate_rows(sh, &lo, &rows);
    if (!keep) {
        long last = (long)sh.q_pos0 + sh.nq - 1;
        long n_hi = last >= sh.w ? (last - sh.w) / sh.s : 0;
        if (n_hi > 16256)
            return fail(FS_ERR_UNSUPPORTED, "without pruning at most 16256 candidate cells");
    }
    const fs::Prior pr{amax, prior_lambda, prior_sigma};
    return from_hip(fs::launch_rerank(sh, q, k, pr, keep, keep_count, keep_width, lo, rows, topk,
                                      idx, score, workspace, workspace ? workspace_bytes : 0,
                                      (hipStream_t)stream),
                    "fs_rerank_topk");
}

fs_status fs_select_workspace_size(const fs_problem* problem, int32_t keep_width, int32_t topk,
                                   size_t* bytes)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    if (keep_width < 0 || keep_width > 4096)
        return fail(FS_ERR_INVALID, "keep_width %d outside [0, 4096]", keep_width);
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    *bytes = fs::select_ws_bytes(sh, keep_width > 0, keep_width, topk);
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_rerank_workspace_size(const fs_problem* problem, int32_t keep_width, size_t* bytes)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    if (keep_width < 0 || keep_width > 4096)
        return fail(FS_ERR_INVALID, "keep_width %d outside [0, 4096]", keep_width);
    *bytes = fs::rerank_ws_bytes(sh, keep_width > 0, keep_width);
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_forest_size(const fs_problem* problem, size_t* bytes)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    if (sh.C > 32768) return fail(FS_ERR_UNSUPPORTED, "FS-B forests hold at most 32768 cells");
    *bytes = fs::forest_bytes(sh);
    return FS_OK;
}

fs_status fs_forest_build(const fs_problem* problem, const float* kbar, const float* amax,
                          const float* tau, void* forest, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (sh.C > 32768) return fail(FS_ERR_UNSUPPORTED, "FS-B forests hold at most 32768 cells");
    FS_PTR(kbar);
    if (!amax) return fail(FS_ERR_INVALID, "amax is NULL");
    if (!forest || ((uintptr_t)forest & 255))
        return fail(FS_ERR_INVALID, "forest must be non-NULL and 256-byte aligned");
    return from_hip(fs::launch_forest_build(sh, kbar, amax, tau, forest, (hipStream_t)stream),
                    "fs_forest_build");
}

fs_status fs_beam_select(const fs_problem* problem, const void* q, const void* k,
                         const void* forest0, const void* forest_tau, int32_t beam, float slack,
                         const float* prior_lambda, const float* prior_sigma, int32_t topk,
                         int32_t* idx, float* score, int32_t* effort, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (sh.C > 32768) return fail(FS_ERR_UNSUPPORTED, "FS-B forests hold at most 32768 cells");
    FS_PTR(q);
    if (k && !aligned16(k)) return fail(FS_ERR_INVALID, "k is not 16-byte aligned");
    if (!forest0 && !forest_tau) return fail(FS_ERR_INVALID, "both forests are NULL");
    if (((uintptr_t)forest0 & 255) || ((uintptr_t)forest_tau & 255))
        return fail(FS_ERR_INVALID, "forests must be 256-byte aligned");
    if (beam < 1 || beam > 64) return fail(FS_ERR_UNSUPPORTED, "beam %d outside [1, 64]", beam);
    if (!(slack >= 0.f) || slack > 3.0e38f)
        return fail(FS_ERR_INVALID, "slack must be finite and >= 0");
    if (prior_lambda && !prior_sigma)
        return fail(FS_ERR_INVALID, "the position prior needs prior_lambda and prior_sigma");
    if (!idx) return fail(FS_ERR_INVALID, "idx is NULL");
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    return from_hip(fs::launch_beam_select(sh, q, k, forest0, forest_tau, beam, (double)slack,
                                           prior_lambda, prior_lambda ? prior_sigma : nullptr,
                                           topk, idx, score, effort, (hipStream_t)stream),
                    "fs_beam_select");
}

fs_status fs_workspace_size(const fs_problem* problem, size_t* bytes)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    *bytes = fs::window_workspace_bytes(sh);
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_window_attn(const fs_problem* problem, const void* q, const void* k, const void* v,
                         float rope_base, void* workspace, size_t ws_bytes, void* o_sr,
                         void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(k); FS_PTR(v); FS_PTR(o_sr); FS_PTR(workspace);
    if (!(rope_base > 1.0f)) return fail(FS_ERR_INVALID, "rope_base must be > 1");
    if (ws_bytes < fs::rope_table_bytes(sh))
        return fail(FS_ERR_INVALID, "workspace of %zu bytes, need %zu", ws_bytes,
                    fs::rope_table_bytes(sh));
    return from_hip(fs::launch_window(sh, q, k, v, (double)rope_base, workspace, o_sr,
                                      (hipStream_t)stream, false, ws_bytes),
                    "fs_window_attn");
}

fs_status fs_window_table(const fs_problem* problem, float rope_base, void* workspace,
                          size_t ws_bytes, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(workspace);
    if (!(rope_base > 1.0f)) return fail(FS_ERR_INVALID, "rope_base must be > 1");
    if (ws_bytes < fs::rope_table_bytes(sh))
        return fail(FS_ERR_INVALID, "workspace of %zu bytes, need %zu", ws_bytes,
                    fs::rope_table_bytes(sh));
    return from_hip(fs::launch_rope_table(sh, (double)rope_base, workspace, (hipStream_t)stream),
                    "fs_window_table");
}

fs_status fs_window_attn_tabled(const fs_problem* problem, const void* q, const void* k,
                                const void* v, void* workspace, size_t ws_bytes, void* o_sr,
                                void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(k); FS_PTR(v); FS_PTR(o_sr); FS_PTR(workspace);
    if (ws_bytes < fs::rope_table_bytes(sh))
        return fail(FS_ERR_INVALID, "workspace of %zu bytes, need %zu", ws_bytes,
                    fs::rope_table_bytes(sh));
    return from_hip(fs::launch_window(sh, q, k, v, 0.0, workspace, o_sr, (hipStream_t)stream,
                                      true, ws_bytes),
                    "fs_window_attn_tabled");
}

fs_status fs_sparse_workspace_size(const fs_problem* problem, size_t* bytes)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    *bytes = fs::sparse_ws_bytes(sh);
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_sparse_attn(const fs_problem* problem, const void* q, const void* k, const void* v,
                         const int32_t* idx, int32_t topk, float rms_eps, void* workspace,
                         size_t ws_bytes, void* o_lr, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(k); FS_PTR(v); FS_PTR(o_lr);
    if (!idx) return fail(FS_ERR_INVALID, "idx is NULL");
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    if (!(rms_eps >= 0.0f)) return fail(FS_ERR_INVALID, "rms_eps must be >= 0");
    if (workspace && ws_bytes < fs::sparse_ws_bytes(sh))
        return fail(FS_ERR_INVALID, "workspace of %zu bytes, need %zu", ws_bytes,
                    fs::sparse_ws_bytes(sh));
    return from_hip(fs::launch_sparse(sh, q, k, v, idx, topk, rms_eps, workspace, o_lr,
                                      (hipStream_t)stream),
                    "fs_sparse_attn");
}

fs_status fs_sparse_attn_combine(const fs_problem* problem, const void* q, const void* k,
                                 const void* v, const int32_t* idx, int32_t topk, float rms_eps,
                                 const void* o_sr, const float* alpha, void* workspace,
                                 size_t ws_bytes, void* o, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(k); FS_PTR(v); FS_PTR(o_sr); FS_PTR(o);
    if (!idx) return fail(FS_ERR_INVALID, "idx is NULL");
    if (!alpha) return fail(FS_ERR_INVALID, "alpha is NULL");
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    if (!(rms_eps >= 0.0f)) return fail(FS_ERR_INVALID, "rms_eps must be >= 0");
    if (workspace && ws_bytes < fs::sparse_ws_bytes(sh))
        return fail(FS_ERR_INVALID, "workspace of %zu bytes, need %zu", ws_bytes,
                    fs::sparse_ws_bytes(sh));
    return from_hip(fs::launch_sparse(sh, q, k, v, idx, topk, rms_eps, workspace, o,
                                      (hipStream_t)stream, o_sr, alpha),
                    "fs_sparse_attn_combine");
}

fs_status fs_sparse_attn_noalloc(const fs_problem* problem, const void* q, const void* k,
                                 const void* v, const int32_t* idx, int32_t topk, float rms_eps,
                                 void* o_lr, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(q); FS_PTR(k); FS_PTR(v); FS_PTR(o_lr);
    if (!idx) return fail(FS_ERR_INVALID, "idx is NULL");
    if (topk < 1 || topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", topk);
    if (!(rms_eps >= 0.0f)) return fail(FS_ERR_INVALID, "rms_eps must be >= 0");
    const size_t need = fs::sparse_ws_bytes(sh);
    if (need > fs::kSparseNoAllocBytes)
        return fail(FS_ERR_UNSUPPORTED,
                    "the split readout needs %zu bytes of scratch, more than the %zu the "
                    "allocation-free call holds", need, fs::kSparseNoAllocBytes);
    void* ws = nullptr;
    if (need > 0) {
        hipError_t e;
        ws = fs::sparse_noalloc_scratch(&e);
        if (!ws) return from_hip(e, "fs_sparse_attn_noalloc: scratch address");
    }
    return from_hip(fs::launch_sparse(sh, q, k, v, idx, topk, rms_eps, ws, o_lr,
                                      (hipStream_t)stream),
                    "fs_sparse_attn_noalloc");
}

}  // extern "C"

namespace {

fs_status check_stream(const fs_stream_config* c, fs::StreamCfg* sc)
{
    if (!c) return fail(FS_ERR_INVALID, "config is NULL");
    if (c->batch < 1 || c->heads < 1) return fail(FS_ERR_INVALID, "batch and heads must be >= 1");
    if ((long)c->batch * c->heads > 65535)
        return fail(FS_ERR_UNSUPPORTED, "batch * heads must be <= 65535");
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(FS_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128", c->head_dim);
    if (c->cell != 32) return fail(FS_ERR_UNSUPPORTED, "cell %d: only 32", c->cell);
    if (c->window < 0 || c->window > (1 << 20))
        return fail(FS_ERR_UNSUPPORTED, "window %d outside [0, 2^20]", c->window);
    if (c->n_recent < 0 || c->budget < 0 || c->n_recent + c->budget < 1 ||
        c->n_recent + c->budget > 1024)
        return fail(FS_ERR_UNSUPPORTED, "n_recent %d + budget %d must be in [1, 1024]",
                    c->n_recent, c->budget);
    if (c->topk < 1 || c->topk > 64) return fail(FS_ERR_UNSUPPORTED, "topk %d outside [1, 64]", c->topk);
    if (c->max_new < 1 || c->max_new > 4096)
        return fail(FS_ERR_UNSUPPORTED, "max_new %d outside [1, 4096]", c->max_new);
    if (c->dtype != FS_F32 && c->dtype != FS_BF16) return fail(FS_ERR_INVALID, "dtype %d", c->dtype);
    if (!(c->rope_base > 1.0f)) return fail(FS_ERR_INVALID, "rope_base must be > 1");
    if (!(c->rms_eps >= 0.0f)) return fail(FS_ERR_INVALID, "rms_eps must be >= 0");
    sc->rope_base = (double)c->rope_base;
    sc->rms_eps = c->rms_eps;
    sc->B = c->batch; sc->H = c->heads; sc->d = c->head_dim; sc->s = c->cell; sc->w = c->window;
    sc->W = c->n_recent; sc->P = c->budget; sc->K = c->topk; sc->max_new = c->max_new;
    sc->bf16 = c->dtype == FS_BF16;
    return FS_OK;
}

fs_status check_state(const fs::StreamLayout& Ly, const void* state, size_t state_bytes)
{
    if (!state) return fail(FS_ERR_INVALID, "state is NULL");
    if (reinterpret_cast<uintptr_t>(state) % 256 != 0)
        return fail(FS_ERR_INVALID, "state is not 256-byte aligned");
    if (state_bytes < Ly.bytes)
        return fail(FS_ERR_INVALID, "state of %zu bytes, need %zu", state_bytes, Ly.bytes);
    return FS_OK;
}

}  // namespace

extern "C" {

fs_status fs_stream_state_size(const fs_stream_config* cfg, size_t* bytes)
{
    fs::StreamCfg sc;
    FS_CHECK(check_stream(cfg, &sc));
    if (!bytes) return fail(FS_ERR_INVALID, "bytes is NULL");
    *bytes = fs::stream_layout(sc).bytes;
    g_err[0] = 0;
    return FS_OK;
}

fs_status fs_stream_reset(const fs_stream_config* cfg, void* state, size_t state_bytes,
                          void* stream)
{
    fs::StreamCfg sc;
    FS_CHECK(check_stream(cfg, &sc));
    const fs::StreamLayout Ly = fs::stream_layout(sc);
    FS_CHECK(check_state(Ly, state, state_bytes));
    return from_hip(fs::launch_stream_reset(sc, Ly, state, (hipStream_t)stream), "fs_stream_reset");
}

fs_status fs_stream_step(const fs_stream_config* cfg, void* state, size_t state_bytes,
                         int64_t pos0, int32_t n_new, const void* q, const void* k,
                         const void* v, const float* alpha, const float* prior_lambda,
                         const float* prior_sigma, void* o, int32_t* idx, void* stream)
{
    fs::StreamCfg sc;
    FS_CHECK(check_stream(cfg, &sc));
    const fs::StreamLayout Ly = fs::stream_layout(sc);
    FS_CHECK(check_state(Ly, state, state_bytes));
    if (n_new < 1 || n_new > sc.max_new)
        return fail(FS_ERR_INVALID, "n_new %d outside [1, max_new = %d]", n_new, sc.max_new);
    if (pos0 < 0 || pos0 + n_new >= ((int64_t)1 << 31))
        return fail(FS_ERR_UNSUPPORTED, "positions %lld .. %lld outside [0, 2^31)",
                    (long long)pos0, (long long)(pos0 + n_new - 1));
    FS_PTR(q); FS_PTR(k); FS_PTR(v); FS_PTR(o);
    if (!alpha) return fail(FS_ERR_INVALID, "alpha is NULL");
    if ((prior_lambda == nullptr) != (prior_sigma == nullptr))
        return fail(FS_ERR_INVALID, "prior_lambda and prior_sigma go together");
    return from_hip(fs::launch_stream_step(sc, Ly, state, pos0, n_new, q, k, v, alpha,
                                           prior_lambda, prior_sigma, o, idx,
                                           (hipStream_t)stream),
                    "fs_stream_step");
}

fs_status fs_combine(const fs_problem* problem, const void* o_sr, const void* o_lr,
                     const float* alpha, void* o, void* stream)
{
    fs::Shape sh;
    FS_CHECK(check_problem(problem, &sh));
    FS_PTR(o_sr); FS_PTR(o_lr); FS_PTR(o);
    if (!alpha) return fail(FS_ERR_INVALID, "alpha is NULL");
    return from_hip(fs::launch_combine(sh, o_sr, o_lr, alpha, o, (hipStream_t)stream),
                    "fs_combine");
}

}  // extern "C"
