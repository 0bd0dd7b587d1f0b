// fs_launch.hpp -- host-side launchers of the FS-L kernels (validated shapes).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fs {

// Records, for fs_last_path(), which kernel path the calling thread's current
// call takes (printf-style).
void note_path(const char* fmt, ...);

// Validated problem shape, as the kernels see it.
struct Shape {
    int B, H, d, N, nq, q_pos0, s, w;
    int bf16;          // 1: bf16 storage, 0: f32 storage
    int C;             // complete cells, N / s
    int64_t qs[3], kvs[3], os[3];
};

// Range of candidate counts spanned by the queries (host helper).
void candidate_rows(const Shape& sh, int* n_lo, int* n_rows);

hipError_t launch_summaries(const Shape& sh, const void* k, float* kbar, float* amax,
                            hipStream_t st);
// ws (nullable, prune_ws_bytes): lets a call with many rows take each cell's
// eviction point once instead of a search per row.
size_t prune_ws_bytes(const Shape& sh);
hipError_t launch_prune(const Shape& sh, const float* amax, int n_lo, int n_rows, int n_recent,
                        int budget, int32_t* keep, int32_t* keep_count, hipStream_t st,
                        void* ws = nullptr, size_t ws_bytes = 0);
// Position prior of eq. 7, lambda_h a_c erf((i - p_c) / (2 sigma_h)): device
// arrays amax [B][H][C], lambda [H], sigma [H]; lambda == nullptr switches it off.
struct Prior {
    const float* amax;
    const float* lambda;
    const float* sigma;
};

// Selection splits a short query range's union over workgroups when ws_bytes >=
// select_ws_bytes (their partial top-K lists, merged by a second kernel).
int select_splits(const Shape& sh, bool pruned, int keep_w);
size_t select_ws_bytes(const Shape& sh, bool pruned, int keep_w, int topk);
hipError_t launch_select(const Shape& sh, const void* q, const float* kbar, const Prior& pr,
                         const int32_t* keep, const int32_t* keep_count, int keep_w, int n_lo,
                         int n_rows, int topk, int32_t* idx, float* score, void* ws,
                         size_t ws_bytes, hipStream_t st);
// Reranking keeps each block's (cell, query) scores in a workspace when ws_bytes
// >= rerank_ws_bytes (pruned: keep != nullptr); otherwise it needs none.
size_t rerank_ws_bytes(const Shape& sh, bool pruned, int keep_w);
hipError_t launch_rerank(const Shape& sh, const void* q, const void* k, const Prior& pr,
                         const int32_t* keep, const int32_t* keep_count, int keep_w, int n_lo,
                         int n_rows, int topk, int32_t* idx, float* score, void* ws,
                         size_t ws_bytes, hipStream_t st);
// Selection over a streaming state's cell pool: keep rows of pool slots (ascending
// cell order), row r of a head (rows_per_head apart) for candidate count
// n_row0 + r; kbar [B*H][M][d], amax and cell_of
// [B*H][M]; lambda == nullptr switches the prior off.  q is [B][H][nq][d] with
// strides qs; queries sit at positions q_pos0 + t.
hipError_t launch_stream_select(int B, int H, int d, bool bf16, const void* q, const int64_t* qs,
                                const float* kbar, const float* amax, const int32_t* cell_of,
                                int M, const float* lambda, const float* sigma, int nq,
                                int64_t q_pos0, int window, int cell, const int32_t* keep,
                                const int32_t* keep_count, int keep_w, int64_t n_row0,
                                int rows_per_head, int topk, int32_t* idx_slot, int32_t* idx_cell,
                                float* score, hipStream_t st);
size_t rope_table_bytes(const Shape& sh);
// Window workspace: the rotation table (rope_table_bytes, filled first unless
// table_ready), then, when ws_bytes >= window_workspace_bytes, the partial states
// of a key range split over window_splits workgroups (short query ranges).
int window_splits(const Shape& sh);
size_t window_ws_bytes(const Shape& sh);
size_t window_workspace_bytes(const Shape& sh);
hipError_t launch_window(const Shape& sh, const void* q, const void* k, const void* v,
                         double rope_base, void* table, void* o_sr, hipStream_t st,
                         bool table_ready, size_t ws_bytes);
// Merge of split attention states (bf16 output with the shape's o strides), with
// the readout's RMSNorm when rms.
// o_sr (nullable): then o = o_sr + alpha[h] * (the merged, RMS-normalised row), eq. 2.
hipError_t launch_split_merge(const Shape& sh, int S, const float* ws_acc, const float2* ws_ml,
                              bool rms, float rms_eps, void* o, hipStream_t st,
                              const void* o_sr = nullptr, const float* alpha = nullptr);
hipError_t launch_rope_table(const Shape& sh, double rope_base, void* table, hipStream_t st);
// Workgroups over which the readout splits each query's cells (1: unsplit), and
// the workspace bytes of their partial softmax states.
int sparse_splits(const Shape& sh);
size_t sparse_ws_bytes(const Shape& sh);
// The allocation-free readout's scratch: its size, and this device's address of
// it (looked up once per device; nullptr and *err set on failure).  The split
// rule launches at most 256 split workgroups of 128 query rows, each row's state
// d fp32 plus (m, l): 16.25 MiB at d = 128, the most any shape needs.
constexpr size_t kSparseNoAllocBytes = (size_t)256 * 128 * (128 * sizeof(float) + 8);
void* sparse_noalloc_scratch(hipError_t* err);

// o_sr (nullable): eq. 2 in the readout's epilogue, o_lr then receives
// o = o_sr + alpha[h] * o_lr (o_lr kept in fp32 until the sum; o may alias o_sr).
hipError_t launch_sparse(const Shape& sh, const void* q, const void* k, const void* v,
                         const int32_t* idx, int topk, float rms_eps, void* ws, void* o_lr,
                         hipStream_t st, const void* o_sr = nullptr,
                         const float* alpha = nullptr);
hipError_t launch_combine(const Shape& sh, const void* o_sr, const void* o_lr, const float* alpha,
                          void* o, hipStream_t st);

// Streaming state (fs_stream.hpp): reset, and one append + attend step.
struct StreamCfg;
struct StreamLayout;
hipError_t launch_stream_reset(const StreamCfg& c, const StreamLayout& Ly, void* state,
                               hipStream_t st);
hipError_t launch_stream_step(const StreamCfg& c, const StreamLayout& Ly, void* state,
                              int64_t pos0, int n_new, const void* q, const void* k,
                              const void* v, const float* alpha, const float* lambda,
                              const float* sigma, void* o, int32_t* idx_cell, hipStream_t st);

// FS-B (section 3.4): forest storage of all (b, h), its construction, and the
// beam search writing S_i like launch_select (ascending cells, -1 padded).
size_t forest_bytes(const Shape& sh);
hipError_t launch_forest_build(const Shape& sh, const float* kbar, const float* amax,
                               const float* tau, void* forest, hipStream_t st);
hipError_t launch_beam_select(const Shape& sh, const void* q, const void* k,
                              const void* forest0, const void* forest_tau, int beam, double slack,
                              const float* prior_lambda, const float* prior_sigma, int topk,
                              int32_t* idx, float* score, int32_t* effort, hipStream_t st);

}  // namespace fs
