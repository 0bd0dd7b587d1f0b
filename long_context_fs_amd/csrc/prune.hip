// prune.hip -- FS-L query-independent prefix pruning (FreeSolo summary,
// section 3.3, eq. 8).
//
// The retained set of a query depends only on its candidate count n, so one
// workgroup builds the row of one n: Recent_W({c < n}) U TopP_{c < n}(a_c).
// The P-th largest priority is found exactly by a bitwise search over the
// 32-bit patterns of a_c (norms are >= 0, so their bit patterns order like the
// values): block-wide counts of "key >= candidate threshold".  Ties at the
// threshold go to the larger cell index.  The row is written in ascending cell
// order.
//
// Rows of up to 8192 candidates keep their keys in registers (cell 256 j + t in
// slot j of thread t): one pass over HBM, one barrier per search step, the
// search starts below the bits every key shares and stops once exactly P keys
// reach the candidate, and the output positions come from one round of per-wave
// ballot counts.  Longer rows use the streaming
// kernel below it.
//
// Many rows (a prefill), given a workspace: row membership has a closed form.
// Cell c is beaten by c' when (a_c', c') > (a_c, c); with E(c) the index of
// the P-th cell beating c (cells in index order; none: never), c is in
// TopP({c' < n}) exactly when c < n <= E(c), since the prefix [0, n) then holds
// fewer than P of its beaters.  One kernel finds E for every cell (a scan of
// the prefix per cell, in LDS chunks), then one workgroup per row compacts
// {c < n : n <= E(c)} U Recent_W with ballots: no per-row search.
#include <climits>

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
            const int total = block_sum(cnt, red);        // block-uniform
            if (total >= budget) {
                thr = cand;
                if (total == budget) break;               // exactly the top budget reach it
            }
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

// Bitwise search and compaction with the row's keys in registers.
template <int KPT>
__global__ __launch_bounds__(kPruneThreads) void prune_reg_kernel(
    const float* __restrict__ amax, int C, int n_lo, int n_rows, int n_recent, int budget,
    int keep_w, int32_t* __restrict__ keep, int32_t* __restrict__ keep_count)
{
    __shared__ int red[2][kPruneWaves];         // double-buffered: one barrier per block sum
    __shared__ int cnt[KPT][kPruneWaves];       // per chunk and wave: kept (then equal) counts
    __shared__ int cnt_eq[KPT][kPruneWaves];
    const int r = blockIdx.x;
    const long bh = blockIdx.y;
    const int n = n_lo + r;
    const uint32_t* key = reinterpret_cast<const uint32_t*>(amax + bh * C);
    int32_t* out = keep + (bh * n_rows + r) * (long)keep_w;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    uint32_t kv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int c = 256 * j + tid;
        kv[j] = c < n ? key[c] : 0u;
    }
    int flip = 0;
    // block sum of a wave-uniform count (ballot popcounts: no lane shuffles)
    auto bsum = [&](int x) {
        if (lane == 0) red[flip][wv] = x;
        __syncthreads();
        int t = 0;
#pragma unroll
        for (int i = 0; i < kPruneWaves; ++i) t += red[flip][i];
        flip ^= 1;
        return t;
    };

    const bool take_all = n <= budget;
    uint32_t thr = 0;
    int n_eq = 0, need_eq = 0;
    if (!take_all) {
        // bits above the highest one in which two valid keys differ are common
        uint32_t k_and = 0xFFFFFFFFu, k_or = 0u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (256 * j + tid < n) {
                k_and &= kv[j];
                k_or |= kv[j];
            }
        }
        // block AND / OR via the two sums of per-bit flags would cost 32 sums;
        // instead reduce the pair through the red buffers directly
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            k_and &= (uint32_t)__shfl_xor((int)k_and, m, kWave);
            k_or |= (uint32_t)__shfl_xor((int)k_or, m, kWave);
        }
        if (lane == 0) {
            red[flip][wv] = (int)k_and;
            red[flip ^ 1][wv] = (int)k_or;
        }
        __syncthreads();
        uint32_t a_all = 0xFFFFFFFFu, o_all = 0u;
#pragma unroll
        for (int i = 0; i < kPruneWaves; ++i) {
            a_all &= (uint32_t)red[flip][i];
            o_all |= (uint32_t)red[flip ^ 1][i];
        }
        __syncthreads();
        const uint32_t diff = a_all ^ o_all;
        int top = 31;
        if (diff == 0u) {
            thr = o_all;                 // every key equal: the ties decide
            top = -1;
        } else {
            top = 31 - __clz(diff);
            thr = top >= 31 ? 0u : (o_all & ~((2u << top) - 1u));
        }
        // largest thr with #{c < n : key_c >= thr} >= budget, i.e. the budget-th largest
        // key; once exactly `budget` keys reach a candidate, they are the top budget
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int c = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) c += __popcll(__ballot(kv[j] >= cand));   // kv = 0 past n, cand >= 1
            const int total = bsum(c);                    // block-uniform
            if (total >= budget) {
                thr = cand;
                if (total == budget) break;
            }
        }
        int gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool valid = 256 * j + tid < n;
            gt += __popcll(__ballot(valid && kv[j] > thr));
            eq += __popcll(__ballot(valid && kv[j] == thr));
        }
        const int n_gt = bsum(gt);
        n_eq = bsum(eq);
        need_eq = budget - n_gt;     // equal keys to keep, those with the largest indices
    }

    // ---- kept flags, then positions in ascending cell order ------------------
    const bool ties = !take_all && n_eq != need_eq;
    if (ties) {
        // rank of each equal key among the equal keys, in cell order
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool is_eq = 256 * j + tid < n && kv[j] == thr;
            const uint64_t m = __ballot(is_eq);
            if (lane == 0) cnt_eq[j][wv] = __popcll(m);
        }
        __syncthreads();
    }
    uint32_t kept_bits = 0u;
    {
        int eq_before = 0;          // equal keys in earlier chunks (ties only)
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int c = 256 * j + tid;
            const bool valid = c < n;
            bool kept = valid && (take_all || kv[j] > thr || c >= n - n_recent);
            if (!take_all && valid && kv[j] == thr) {
                if (!ties) {
                    kept = true;
                } else {
                    const uint64_t m = __ballot(kv[j] == thr && valid);
                    int rank = eq_before + lanes_below(m);
#pragma unroll
                    for (int i = 0; i < kPruneWaves; ++i) rank += i < wv ? cnt_eq[j][i] : 0;
                    kept = kept || rank >= n_eq - need_eq;
                }
            }
            if (ties) {
#pragma unroll
                for (int i = 0; i < kPruneWaves; ++i) eq_before += cnt_eq[j][i];
            }
            kept_bits |= (uint32_t)kept << j;
            const uint64_t km = __ballot(kept);
            if (lane == 0) cnt[j][wv] = __popcll(km);
        }
    }
    __syncthreads();
    int written = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool kept = (kept_bits >> j) & 1u;
        const uint64_t km = __ballot(kept);
        int pos = written + lanes_below(km);
#pragma unroll
        for (int i = 0; i < kPruneWaves; ++i) {
            pos += i < wv ? cnt[j][i] : 0;
            written += cnt[j][i];
        }
        if (kept) out[pos] = 256 * j + tid;
    }
    for (int t = written + tid; t < keep_w; t += kPruneThreads) out[t] = -1;
    if (tid == 0) keep_count[bh * n_rows + r] = written;
}

// E(c) for the cells c < n_max of each (b, h): the index of the budget-th cell
// beating c in index order, or INT_MAX.  A workgroup stages the head's keys in
// LDS and its waves take kEvictCells cells each: a wave walks the prefix 64
// cells at a time (lane l takes cell r0 + l), counts that round's beaters with a
// ballot, and in the round where the running count reaches `budget` picks the
// beater of the remaining rank from the ballot mask.
constexpr int kEvictCells = 4;                  // cells per wave
constexpr int kEvictMaxCells = 8192;

__global__ __launch_bounds__(kPruneThreads) void prune_evict_kernel(
    const float* __restrict__ amax, int C, int n_max, int budget, int32_t* __restrict__ evict)
{
    __shared__ uint32_t kbuf[kEvictMaxCells];
    const long bh = blockIdx.y;
    const uint32_t* key = reinterpret_cast<const uint32_t*>(amax + bh * C);
    for (int t = threadIdx.x; t < n_max; t += kPruneThreads) kbuf[t] = key[t];
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c0 = (blockIdx.x * kPruneWaves + wv) * kEvictCells;
    for (int ci = 0; ci < kEvictCells; ++ci) {
        const int c = c0 + ci;                           // wave-uniform
        if (c >= n_max) break;
        const uint32_t kc = kbuf[c];
        int total = 0, e = INT_MAX;
        for (int r0 = 0; r0 < n_max; r0 += kWave) {
            const int cp = r0 + lane;
            bool beat = false;
            if (cp < n_max) {
                const uint32_t kp = kbuf[cp];
                beat = kp > kc || (kp == kc && cp > c);
            }
            uint64_t m = __ballot(beat);
            const int cnt = __popcll(m);
            if (total + cnt >= budget) {                 // wave-uniform
                for (int k = budget - total; k > 1; --k) m &= m - 1;   // drop lower beaters
                e = r0 + __ffsll((long long)m) - 1;
                break;
            }
            total += cnt;
        }
        if (lane == 0) evict[bh * n_max + c] = e;
    }
}

// Rows n = n_lo + r for kRowsPerBlock consecutive r from E: {c < n : n <= E(c)}
// U {n - n_recent <= c < n}, ascending, by per-wave ballots (cell 256 j + t in
// slot j of thread t; E read once for the block's rows).
constexpr int kRowsPerBlock = 8;

template <int KPT>
__global__ __launch_bounds__(kPruneThreads) void prune_rows_kernel(
    const int32_t* __restrict__ evict, int n_max, int n_lo, int n_rows, int n_recent, int keep_w,
    int32_t* __restrict__ keep, int32_t* __restrict__ keep_count)
{
    __shared__ int cnt[KPT][kPruneWaves];
    const long bh = blockIdx.y;
    const int32_t* E = evict + bh * n_max;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r0 = blockIdx.x * kRowsPerBlock;
    int ev[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int c = 256 * j + tid;
        ev[j] = c < n_max ? E[c] : 0;
    }
    for (int rr = 0; rr < kRowsPerBlock; ++rr) {
        const int r = r0 + rr;
        if (r >= n_rows) break;                          // block-uniform
        const int n = n_lo + r;
        int32_t* out = keep + (bh * n_rows + r) * (long)keep_w;
        uint32_t kept_bits = 0u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int c = 256 * j + tid;
            const bool kept = c < n && (n <= ev[j] || c >= n - n_recent);
            kept_bits |= (uint32_t)kept << j;
            const uint64_t km = __ballot(kept);
            if (lane == 0) cnt[j][wv] = __popcll(km);
        }
        __syncthreads();
        int written = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool kept = (kept_bits >> j) & 1u;
            const uint64_t km = __ballot(kept);
            int pos = written + lanes_below(km);
#pragma unroll
            for (int i = 0; i < kPruneWaves; ++i) {
                pos += i < wv ? cnt[j][i] : 0;
                written += cnt[j][i];
            }
            if (kept) out[pos] = 256 * j + tid;
        }
        for (int t = written + tid; t < keep_w; t += kPruneThreads) out[t] = -1;
        if (tid == 0) keep_count[bh * n_rows + r] = written;
        __syncthreads();                                 // cnt is rewritten by the next row
    }
}

// Workspace of the many-row path: E per cell below the largest candidate count.
size_t prune_ws_bytes(const Shape& sh)
{
    int n_lo, n_rows;
    candidate_rows(sh, &n_lo, &n_rows);
    const long n_max = n_rows > 0 ? n_lo + n_rows - 1 : 0;
    return (size_t)sh.B * sh.H * n_max * sizeof(int32_t);
}

// The closed form pays one scan of the prefix per cell; the per-row search pays
// a bitwise search per row.  With rows at least a sixteenth of the cells the
// scan is the cheaper.
static bool prune_by_evict(int n_rows, int n_max)
{
    return n_rows >= 64 && 16L * n_rows >= n_max && n_max <= kEvictMaxCells;
}

hipError_t launch_prune(const Shape& sh, const float* amax, int n_lo, int n_rows, int n_recent,
                        int budget, int32_t* keep, int32_t* keep_count, hipStream_t st, void* ws,
                        size_t ws_bytes)
{
    if (n_rows == 0) return hipSuccess;
    dim3 grid((unsigned)n_rows, (unsigned)(sh.B * sh.H)), block(kPruneThreads);
    const int n_max = n_lo + n_rows - 1;
    const int kpt = (n_max + kPruneThreads - 1) / kPruneThreads;
    if (ws && ws_bytes >= prune_ws_bytes(sh) && budget > 0 && prune_by_evict(n_rows, n_max)) {
        int32_t* evict = static_cast<int32_t*>(ws);
        constexpr int per_block = kPruneWaves * kEvictCells;
        dim3 egrid((unsigned)((n_max + per_block - 1) / per_block), (unsigned)(sh.B * sh.H));
        hipLaunchKernelGGL(prune_evict_kernel, egrid, block, 0, st, amax, sh.C, n_max, budget,
                           evict);
        dim3 rgrid((unsigned)((n_rows + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)(sh.B * sh.H));
#define FS_PRUNE_ROWS(K)                                                                        \
        hipLaunchKernelGGL((prune_rows_kernel<K>), rgrid, block, 0, st, evict, n_max, n_lo,     \
                           n_rows, n_recent, n_recent + budget, keep, keep_count)
        if (kpt <= 4) FS_PRUNE_ROWS(4);
        else if (kpt <= 8) FS_PRUNE_ROWS(8);
        else if (kpt <= 16) FS_PRUNE_ROWS(16);
        else FS_PRUNE_ROWS(32);
#undef FS_PRUNE_ROWS
        return hipGetLastError();
    }
#define FS_PRUNE_REG(K)                                                                         \
    hipLaunchKernelGGL((prune_reg_kernel<K>), grid, block, 0, st, amax, sh.C, n_lo, n_rows,     \
                       n_recent, budget, n_recent + budget, keep, keep_count)
    if (kpt <= 4) FS_PRUNE_REG(4);
    else if (kpt <= 8) FS_PRUNE_REG(8);
    else if (kpt <= 16) FS_PRUNE_REG(16);
    else if (kpt <= 32) FS_PRUNE_REG(32);
    else
        hipLaunchKernelGGL(prune_kernel, grid, block, 0, st, amax, sh.C, n_lo, n_rows, n_recent,
                           budget, n_recent + budget, keep, keep_count);
#undef FS_PRUNE_REG
    return hipGetLastError();
}

}  // namespace fs
