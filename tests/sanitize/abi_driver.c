/*
 * abi_driver.c -- drives the host side of the C ABI (include/fs.h) for a build
 * of the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize_cpu.py): every entry point with arguments its host-side
 * validation must refuse before anything is enqueued, and the host helpers
 * (candidate rows, workspace and state sizes) on valid shapes.  No GPU is used:
 * no call here reaches a kernel launch.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fs.h"

static int g_fail = 0;

static void expect(fs_status got, fs_status want, const char* what)
{
    if (got != want) {
        printf("%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, fs_last_error());
        g_fail = 1;
    }
    (void)fs_status_string(got);
    (void)fs_last_error();
    (void)fs_last_path();
}

static fs_problem prob(int B, int H, int d, int N, int nq, int q0, int w, int dtype)
{
    fs_problem p;
    memset(&p, 0, sizeof(p));
    p.batch = B; p.heads = H; p.head_dim = d; p.n_ctx = N; p.n_q = nq; p.q_pos0 = q0;
    p.cell = 32; p.window = w; p.dtype = dtype;
    p.q_stride[0] = (int64_t)H * nq * d; p.q_stride[1] = (int64_t)nq * d; p.q_stride[2] = d;
    p.kv_stride[0] = (int64_t)H * N * d; p.kv_stride[1] = (int64_t)N * d; p.kv_stride[2] = d;
    p.o_stride[0] = (int64_t)H * nq * d; p.o_stride[1] = (int64_t)nq * d; p.o_stride[2] = d;
    return p;
}

int main(void)
{
    static char buf[1 << 16] __attribute__((aligned(256)));
    void* x = buf;                      /* any aligned, non-NULL address: nothing runs */
    int32_t* ix = (int32_t*)buf;
    float* fx = (float*)buf;
    size_t n = 0;
    int32_t lo = 0, rows = 0;
    const fs_problem good = prob(2, 3, 64, 4096, 1000, 3000, 512, FS_BF16);
    const fs_problem big = prob(1, 8, 128, 262144, 256, 262144 - 256, 512, FS_BF16);

    /* host helpers on valid shapes */
    expect(fs_prune_rows(&good, &lo, &rows), FS_OK, "prune_rows");
    expect(fs_workspace_size(&good, &n), FS_OK, "workspace_size");
    expect(fs_sparse_workspace_size(&big, &n), FS_OK, "sparse_workspace_size");
    expect(fs_select_workspace_size(&big, 512, 32, &n), FS_OK, "select_workspace_size");
    expect(fs_rerank_workspace_size(&good, 64, &n), FS_OK, "rerank_workspace_size");
    expect(fs_forest_size(&good, &n), FS_OK, "forest_size");
    fs_stream_config sc;
    memset(&sc, 0, sizeof(sc));
    sc.batch = 1; sc.heads = 8; sc.head_dim = 128; sc.cell = 32; sc.window = 512; sc.n_recent = 0;
    sc.budget = 512; sc.topk = 32; sc.max_new = 256; sc.dtype = FS_BF16; sc.rope_base = 10000.f;
    sc.rms_eps = 1e-6f;
    expect(fs_stream_state_size(&sc, &n), FS_OK, "stream_state_size");

    /* refused before any launch: NULL problem, bad shapes, bad pointers */
    fs_problem bad = good;
    expect(fs_cell_summaries(NULL, x, fx, fx, NULL), FS_ERR_INVALID, "summaries NULL problem");
    bad.head_dim = 96;
    expect(fs_cell_summaries(&bad, x, fx, fx, NULL), FS_ERR_UNSUPPORTED, "summaries d 96");
    bad = good; bad.cell = 16;
    expect(fs_window_attn(&bad, x, x, x, 1e4f, x, 1 << 16, x, NULL), FS_ERR_UNSUPPORTED, "cell 16");
    bad = good; bad.q_pos0 = 4000;
    expect(fs_sparse_attn(&bad, x, x, x, ix, 8, 1e-6f, NULL, 0, x, NULL), FS_ERR_INVALID, "q range");
    bad = good; bad.q_stride[2] = 3;
    expect(fs_combine(&bad, x, x, fx, x, NULL), FS_ERR_INVALID, "row stride");
    bad = good; bad.reserved = 1;
    expect(fs_select_topk(&bad, x, fx, NULL, NULL, NULL, NULL, NULL, 0, 8, ix, NULL, NULL, 0, NULL),
           FS_ERR_INVALID, "reserved");
    expect(fs_select_topk(&good, x, fx, NULL, NULL, NULL, NULL, NULL, 0, 65, ix, NULL, NULL, 0, NULL),
           FS_ERR_UNSUPPORTED, "topk 65");
    expect(fs_select_topk(&good, x, fx, NULL, fx, NULL, NULL, NULL, 0, 8, ix, NULL, NULL, 0, NULL),
           FS_ERR_INVALID, "prior without sigma");
    expect(fs_rerank_topk(&good, x, x, NULL, NULL, NULL, ix, NULL, 8, 8, ix, NULL, NULL, 0, NULL),
           FS_ERR_INVALID, "keep without keep_count");
    expect(fs_prune_prefix(&good, fx, 0, 0, ix, ix, NULL, 0, NULL), FS_ERR_UNSUPPORTED, "budget 0");
    expect(fs_prune_prefix(&good, fx, 0, 8, ix, ix, x, 4, NULL), FS_ERR_INVALID,
           "small prune workspace");
    expect(fs_prune_workspace_size(&good, NULL), FS_ERR_INVALID, "prune ws NULL");
    expect(fs_sparse_attn(&good, (char*)x + 4, x, x, ix, 8, 1e-6f, NULL, 0, x, NULL),
           FS_ERR_INVALID, "misaligned q");
    expect(fs_sparse_attn(&good, x, x, x, ix, 8, -1.f, NULL, 0, x, NULL), FS_ERR_INVALID, "eps");
    expect(fs_sparse_attn(&big, x, x, x, ix, 8, 1e-6f, x, 16, x, NULL), FS_ERR_INVALID,
           "small workspace");
    expect(fs_sparse_attn_noalloc(&good, x, x, x, NULL, 8, 1e-6f, x, NULL), FS_ERR_INVALID,
           "noalloc NULL idx");
    expect(fs_window_attn(&good, x, x, NULL, 1e4f, x, 1 << 16, x, NULL), FS_ERR_INVALID, "NULL v");
    expect(fs_forest_build(&good, fx, fx, NULL, NULL, NULL), FS_ERR_INVALID, "NULL forest");
    expect(fs_beam_select(&good, x, NULL, NULL, NULL, 8, 1.f, NULL, NULL, 8, ix, NULL, NULL,
                          NULL),
           FS_ERR_INVALID, "no forest");
    expect(fs_beam_select(&good, x, NULL, x, NULL, 65, 1.f, NULL, NULL, 8, ix, NULL, NULL, NULL),
           FS_ERR_UNSUPPORTED, "beam 65");
    expect(fs_beam_select(&good, x, (const char*)x + 2, x, NULL, 8, 1.f, NULL, NULL, 8, ix, NULL,
                          NULL, NULL),
           FS_ERR_INVALID, "misaligned keys");
    sc.max_new = 0;
    expect(fs_stream_state_size(&sc, &n), FS_ERR_UNSUPPORTED, "stream max_new 0");
    expect(fs_stream_step(&sc, x, 1 << 16, 0, 1, x, x, x, fx, NULL, NULL, x, NULL, NULL),
           FS_ERR_UNSUPPORTED, "stream step bad config");
    puts(g_fail ? "abi driver: FAILED" : "abi driver: done");
    return g_fail;
}
