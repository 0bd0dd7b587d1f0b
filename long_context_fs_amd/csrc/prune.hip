// prune.hip -- FS-L query-independent prefix pruning (FreeSolo summary,
// section 3.3, eq. 8).
//
// The retained set of a query depends only on its candidate count n, so one
// workgroup builds the row of one n: Recent_W({c < n}) U TopP_{c < n}(a_c).
// The P-th largest priority is found exactly by a bitwise search over the
// 32-bit patterns of a_c (norms are >= 0, so their bit patterns order like the
// values), 32 block-wide counts of "key >= candidate threshold".  Ties at the
// threshold go to the larger cell index.  The row is then written in ascending
// cell order by a chunked block prefix sum (wave ballot + popcount).
#include "fs_device.hpp"
#include "fs_launch.hpp"

namespace fs {

constexpr int kPruneThreads = 256;
constexpr int kPruneWaves = kPruneThreads / kWave;

// Block-wide sum of one int per thread.
__device__ __forceinline__ int block_sum(int x, int* red)
{
    x = wave_sum_int(x);
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wv] = x;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < kPruneWaves; ++i) t += red[i];
    return t;
}

// Exclusive block prefix of one flag per thread; *total gets the block count.
__device__ __forceinline__ int block_prefix(bool flag, int* red, int* total)
{
    const uint64_t m = __ballot(flag);
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wv] = __popcll(m);
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kPruneWaves; ++i) {
        before += (i < wv) ? red[i] : 0;
        all += red[i];
    }
    *total = all;
    return before + lanes_below(m);
}

__global__ __launch_bounds__(kPruneThreads) void prune_kernel(
    const float* __restrict__ amax, int C, int n_lo, int n_rows, int n_recent, int budget,
    int keep_w, int32_t* __restrict__ keep, int32_t* __restrict__ keep_count)
{
    __shared__ int red[kPruneWaves];
    const int r = blockIdx.x;
    const long bh = blockIdx.y;
    const int n = n_lo + r;
    const uint32_t* key = reinterpret_cast<const uint32_t*>(amax + bh * C);
    int32_t* out = keep + (bh * n_rows + r) * (long)keep_w;
    const int tid = threadIdx.x;

    const bool take_all = n <= budget;
    uint32_t thr = 0;
    int n_eq = 0, need_eq = 0;
    if (!take_all) {
        // Largest thr with #{c < n : key_c >= thr} >= budget, i.e. the budget-th largest key.
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int cnt = 0;
            for (int c = tid; c < n; c += kPruneThreads) cnt += key[c] >= cand;
            if (block_sum(cnt, red) >= budget) thr = cand;
        }
        int gt = 0, eq = 0;
        for (int c = tid; c < n; c += kPruneThreads) {
            gt += key[c] > thr;
            eq += key[c] == thr;
        }
        const int n_gt = block_sum(gt, red);
        n_eq = block_sum(eq, red);
        need_eq = budget - n_gt;     // equal keys to keep, those with the largest indices
    }

    int written = 0, eq_seen = 0;
    for (int c0 = 0; c0 < n; c0 += kPruneThreads) {
        const int c = c0 + tid;
        const bool in = c < n;
        const uint32_t kc = in ? key[c] : 0u;
        const bool is_eq = in && !take_all && kc == thr;
        int n_eq_chunk;
        const int eq_rank = eq_seen + block_prefix(is_eq, red, &n_eq_chunk);
        const bool kept = in && (take_all || kc > thr || c >= n - n_recent ||
                                 (is_eq && eq_rank >= n_eq - need_eq));
        int n_kept;
        const int pos = written + block_prefix(kept, red, &n_kept);
        if (kept) out[pos] = c;
        written += n_kept;
        eq_seen += n_eq_chunk;
    }
    for (int t = written + tid; t < keep_w; t += kPruneThreads) out[t] = -1;
    if (tid == 0) keep_count[bh * n_rows + r] = written;
}

hipError_t launch_prune(const Shape& sh, const float* amax, int n_lo, int n_rows, int n_recent,
                        int budget, int32_t* keep, int32_t* keep_count, hipStream_t st)
{
    if (n_rows == 0) return hipSuccess;
    dim3 grid((unsigned)n_rows, (unsigned)(sh.B * sh.H)), block(kPruneThreads);
    hipLaunchKernelGGL(prune_kernel, grid, block, 0, st, amax, sh.C, n_lo, n_rows, n_recent,
                       budget, n_recent + budget, keep, keep_count);
    return hipGetLastError();
}

}  // namespace fs
