// select.hip -- cell scoring and per-query top-K (FreeSolo summary, section 3.3,
// eq. 7, with its position prior when lambda is given; the selected set S_i of
// eq. 9), token-level reranking (section 3.4, eq. 12), and the selection over a
// streaming state's cell pool.
//
// One wavefront per query row.  The unrotated query is staged in LDS; each lane
// scores candidate cells c (from the keep row of the query's candidate count,
// or every c < n_i without pruning) as the fp32 dot q . kbar_c.  Ranking uses
// the unscaled dot (1/sqrt(d) > 0 does not change the order and must not merge
// neighbouring scores); the reported score is dot / sqrt(d).  The K-th largest
// key is found exactly by a bitwise search with ballot counts, ties at the
// threshold go to the larger cell, and the chosen cells are written ascending.
//
// Candidate lists up to 528 cells: MFMA kernel.  A workgroup
// owns 64 consecutive queries (4 wavefronts x 16); they span at most three
// candidate counts, so their candidates are the union of at most three keep
// rows (or the prefix [0, n) without pruning), built in LDS with a bitmap.
// kbar rows of the union are staged 32 at a time, each fp32 value split into
// three bf16 parts hi + mid + lo (24 significant bits); q is exact in bf16, so
// three exact-product MFMAs with fp32 accumulation give fp32-accurate scores.
// The scores stay in the MFMA output registers as order-preserving keys: the
// four lanes n, n+16, n+32, n+48 hold query n's union slots 16 bb + 4 g + r.
// The K-th largest key is found by a bitwise search over those four lanes
// (gfx950 row swaps for the sums), starting below the bits all valid keys share
// and stopping once exactly K keys reach the candidate; the chosen cells are
// written in slot order from packed prefix counts over the four lanes.  For
// short query ranges the union can be split over workgroups of 64 slots, whose
// top-K lists a merge kernel ranks again.  f32 storage runs the same kernel with
// q and kbar kept in fp32 and the scores from the fp32 matrix product.
//
// Reranking (eq. 12) scores each candidate cell by the log-sum-exp of its 32
// token logits: 32x32x16 MFMA over two-cell key tiles for 128 queries per
// workgroup (scores through a caller workspace), or 16x16x32 for 64 queries.
#include "fs_device.hpp"
#include "fs_launch.hpp"
#include "mfma_tile.hpp"

namespace fs {

constexpr int kSelWaves = 4;

__device__ __forceinline__ float key_to_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exact top-K of one query (one wavefront) over the order-preserving keys
// s_key[0..n_cand) in LDS.  The K-th largest key thr is found by a bitwise
// search whose counts are ballots (wave-uniform, no lane shuffles); bits that all
// keys share are fixed from the start, and the search stops as soon as exactly K
// keys reach the candidate (that set is then the top K).  Of the keys equal to
// thr, the last ones in list order are kept (the lists are ascending in cell
// index, so ties go to the larger cell).  The chosen entries are handed over in
// list order, emit(pos, j, key) for output position pos = 0 .. min(K, n_cand) - 1;
// pad(t) is called for the positions t from min(K, n_cand) to K - 1.
template <class Emit, class Pad>
__device__ __forceinline__ void row_topk_write(const uint32_t* s_key, int n_cand, int topk,
                                               int lane, Emit emit, Pad pad)
{
    const int kq = n_cand < topk ? n_cand : topk;
    // up to 1024 keys are held in registers (0 pads: every finite score's key is
    // >= 2^23, and every candidate threshold is >= 1), beyond that they are read
    // from LDS at each step
    constexpr int kRegKeys = 16;
    const bool in_regs = n_cand <= kRegKeys * kWave;
    uint32_t kr[kRegKeys];
#pragma unroll
    for (int r = 0; r < kRegKeys; ++r) {
        const int j = lane + r * kWave;
        kr[r] = in_regs && j < n_cand ? s_key[j] : 0u;
    }
    auto count_ge = [&](uint32_t t) {        // #{j : s_key[j] >= t}, wave-uniform
        int c = 0;
        if (in_regs) {
#pragma unroll
            for (int r = 0; r < kRegKeys; ++r) c += __popcll(__ballot(kr[r] >= t));
        } else {
            for (int j0 = 0; j0 < n_cand; j0 += kWave) {
                const int j = j0 + lane;
                c += __popcll(__ballot(j < n_cand && s_key[j] >= t));
            }
        }
        return c;
    };
    uint32_t thr = 0;
    if (kq > 0) {
        uint32_t k_and = 0xFFFFFFFFu, k_or = 0u;
        for (int j = lane; j < n_cand; j += kWave) {
            k_and &= s_key[j];
            k_or |= s_key[j];
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            k_and &= (uint32_t)__shfl_xor((int)k_and, m, kWave);
            k_or |= (uint32_t)__shfl_xor((int)k_or, m, kWave);
        }
        const uint32_t diff = k_and ^ k_or;
        if (diff == 0u) {
            thr = k_or;                      // every key equal
        } else {
            const int hb = 31 - __clz(diff);
            thr = k_or & ~(hb >= 31 ? 0xFFFFFFFFu : (2u << hb) - 1u);
            for (int bit = hb; bit >= 0; --bit) {
                const uint32_t t = thr | (1u << bit);
                const int c = count_ge(t);
                if (c >= kq) {
                    thr = t;
                    if (c == kq) break;      // exactly the top kq reach t
                }
            }
        }
    }
    int n_gt = 0, n_eq = 0;
    for (int j0 = 0; j0 < n_cand; j0 += kWave) {
        const int j = j0 + lane;
        n_gt += __popcll(__ballot(j < n_cand && s_key[j] > thr));
        n_eq += __popcll(__ballot(j < n_cand && s_key[j] == thr));
    }
    const int need_eq = kq - n_gt;

    int written = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n_cand && kq > 0; j0 += kWave) {
        const int j = j0 + lane;
        const bool in = j < n_cand;
        const uint32_t kj = in ? s_key[j] : 0u;
        const bool is_eq = in && kj == thr;
        const uint64_t me = __ballot(is_eq);
        const int eq_rank = eq_seen + lanes_below(me);
        const bool kept = in && (kj > thr || (is_eq && eq_rank >= n_eq - need_eq));
        const uint64_t mk = __ballot(kept);
        if (kept) emit(written + lanes_below(mk), j, kj);
        written += __popcll(mk);
        eq_seen += __popcll(me);
    }
    for (int t = kq + lane; t < topk; t += kWave) pad(t);
}

// eq. 7's prior for the query at position i and cell c of head h (row bh of amax):
// lambda_h a_c erf((i - p_c) / (2 sigma_h)), p_c = (c + 1/2) s.  i - c s is exact in
// fp32 below 2^24 tokens; beyond, erf has long saturated for any sigma that small.
__device__ __forceinline__ float prior_term(const Prior& pr, long bh, int h, int C, long i, int c,
                                            int cell)
{
    const float a = pr.amax[bh * C + c];
    const float delta = (float)(i - (long)c * cell) - 0.5f * (float)cell;
    return pr.lambda[h] * a * erff(delta / (2.f * pr.sigma[h]));
}

// RERANK: score a cell by eq. 12's log-sum-exp of its token logits (k, kvs*)
// instead of eq. 7's mean-key dot (kbar).
template <class E, int D, bool RERANK>
__global__ __launch_bounds__(kSelWaves * kWave) void select_topk_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ kbar, const typename E::storage* __restrict__ k, int64_t kvs0,
    int64_t kvs1, int64_t kvs2, Prior pr, int H, int C, int nq, int q_pos0, int window,
    int cell, const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_count, int keep_w,
    int n_lo, int n_rows, int topk, int cap, float inv_sqrt_d, int32_t* __restrict__ idx,
    float* __restrict__ score)
{
    extern __shared__ uint32_t smem[];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    float* s_q = reinterpret_cast<float*>(smem) + wv * D;
    uint32_t* s_key = smem + waves * D + wv * cap;

    const long row = (long)blockIdx.x * waves + wv;
    const long bh = blockIdx.y;
    const bool active = row < nq;       // inactive waves still reach the barrier
    const int h = (int)(bh % H), b = (int)(bh / H);
    const long i = (long)q_pos0 + (active ? row : 0);
    const int n = active ? n_candidates(i, window, cell, C) : 0;

    const int32_t* cand = nullptr;
    int n_cand = n;
    if (keep != nullptr) {
        n_cand = 0;
        if (n > 0) {
            const long kr = bh * n_rows + (n - n_lo);
            cand = keep + kr * keep_w;
            n_cand = keep_count[kr];
        }
    }
    if (active) {
        const typename E::storage* qrow = q + b * qs0 + h * qs1 + row * qs2;
        for (int e = lane; e < D; e += kWave) s_q[e] = load1<E>(qrow + e);
    }
    __syncthreads();

    if constexpr (RERANK) {
        // one candidate cell at a time: lane t < s takes token t of the cell
        const typename E::storage* kh = k + b * kvs0 + h * kvs1;
        for (int j = 0; j < n_cand; ++j) {
            const int c = cand ? cand[j] : j;
            float lg = -INFINITY;
            if (lane < cell) {
                const typename E::storage* kr = kh + ((long)c * cell + lane) * kvs2;
                float dot = 0.f;
                for (int e = 0; e < D; ++e) dot = fmaf(s_q[e], load1<E>(kr + e), dot);
                lg = dot * inv_sqrt_d;
            }
            const float m = wave_max(lg);
            const float z = wave_sum(lane < cell ? expf(lg - m) : 0.f);
            const float r = m + logf(z) + (pr.lambda ? prior_term(pr, bh, h, C, i, c, cell) : 0.f);
            if (lane == 0) s_key[j] = float_key(r);
        }
    } else {
        const float* kb_head = kbar + bh * (long)C * D;
        for (int j = lane; j < n_cand; j += kWave) {
            const int c = cand ? cand[j] : j;
            const float* kb = kb_head + (long)c * D;
            float dot = 0.f;
#pragma unroll 8
            for (int e = 0; e < D; e += 4) {
                const float4 kv = *reinterpret_cast<const float4*>(kb + e);
                dot = fmaf(s_q[e], kv.x, dot);
                dot = fmaf(s_q[e + 1], kv.y, dot);
                dot = fmaf(s_q[e + 2], kv.z, dot);
                dot = fmaf(s_q[e + 3], kv.w, dot);
            }
            // ranked by the unscaled dot without the prior (1/sqrt(d) > 0 keeps the order)
            s_key[j] = float_key(pr.lambda ? fmaf(dot, inv_sqrt_d,
                                                  prior_term(pr, bh, h, C, i, c, cell))
                                           : dot);
        }
    }
    __syncthreads();
    if (!active) return;

    int32_t* out_i = idx + (bh * nq + row) * (long)topk;
    float* out_s = score ? score + (bh * nq + row) * (long)topk : nullptr;
    const float out_scale = RERANK || pr.lambda ? 1.f : inv_sqrt_d;
    row_topk_write(
        s_key, n_cand, topk, lane,
        [&](int pos, int j, uint32_t kj) {
            out_i[pos] = cand ? cand[j] : j;
            if (out_s) out_s[pos] = key_to_float(kj) * out_scale;
        },
        [&](int t) {
            out_i[t] = -1;
            if (out_s) out_s[t] = 0.f;
        });
}


// Selection over a streaming state's cell pool (eq. 7 on the cells FS-L still
// holds).  The keep row of a query lists pool slots in ascending cell order;
// kbar, a_c and the cell index are stored per slot.  QPB queries per workgroup
// (1 for a decode step, 4 otherwise): the query's threads take one candidate per
// group of D / 8 lanes (8 dims a lane, q in registers), so a candidate's kbar row
// is one coalesced read and many rows are in flight; the dot is finished by a
// butterfly over the group.  One wavefront per query then ranks the keys as the
// row-wise kernel does.  idx_slot receives slots (what the readout gathers),
// idx_cell (optional) the same choice as cell indices.
template <class E, int D, int QPB>
__global__ __launch_bounds__(256) void stream_select_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ kbar, const float* __restrict__ amax,
    const int32_t* __restrict__ cell_of, int M, const float* __restrict__ lambda,
    const float* __restrict__ sigma, int H, int nq, int64_t q_pos0, int window, int cell,
    const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_count, int keep_w,
    int64_t n_row0, int rows_per_head, int topk, float inv_sqrt_d, int32_t* __restrict__ idx_slot,
    int32_t* __restrict__ idx_cell, float* __restrict__ score)
{
    constexpr int TPQ = 256 / QPB;          // threads per query
    constexpr int LPC = D / 8;              // lanes per candidate
    constexpr int CPI = TPQ / LPC;          // candidates per iteration
    constexpr int UNR = QPB == 1 ? 16 : 4;  // candidate rows in flight per lane group
    extern __shared__ uint32_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int qi = tid / TPQ, tq = tid % TPQ;
    const int grp = tq / LPC, gl = tq % LPC;
    uint32_t* s_key = smem + qi * keep_w;
    int32_t* s_cand = reinterpret_cast<int32_t*>(smem + QPB * keep_w) + qi * keep_w;

    const long row = (long)blockIdx.x * QPB + qi;
    const long bh = blockIdx.y;
    const bool active = row < nq;           // inactive queries still reach the barrier
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int64_t i = q_pos0 + (active ? row : 0);
    const int64_t n = i < window ? 0 : (i - window) / cell;
    const long kr = bh * rows_per_head + (long)(n - n_row0);
    const int32_t* cand = keep + kr * keep_w;
    const int n_cand = active ? keep_count[kr] : 0;
    for (int j = tq; j < n_cand; j += TPQ) s_cand[j] = cand[j];   // the keep row, once
    float qv[8];
    {
        const typename E::storage* qrow = q + b * qs0 + h * qs1 + (active ? row : 0) * qs2 + gl * 8;
        if constexpr (E::kPer16B == 8) {
            load16<E>(qrow, qv);
        } else {
            load16<E>(qrow, qv);
            load16<E>(qrow + 4, qv + 4);
        }
    }
    const float* kb_head = kbar + bh * (long)M * D + gl * 8;
    __syncthreads();
    for (int j0 = 0; j0 < n_cand; j0 += CPI * UNR) {
        float dot[UNR];
        int slot[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {     // UNR candidates' rows in flight
            const int j = j0 + u * CPI + grp;
            slot[u] = j < n_cand ? s_cand[j] : 0;
            const float4 x0 = *reinterpret_cast<const float4*>(kb_head + (long)slot[u] * D);
            const float4 x1 = *reinterpret_cast<const float4*>(kb_head + (long)slot[u] * D + 4);
            float d0 = qv[0] * x0.x;
            d0 = fmaf(qv[1], x0.y, d0);
            d0 = fmaf(qv[2], x0.z, d0);
            d0 = fmaf(qv[3], x0.w, d0);
            d0 = fmaf(qv[4], x1.x, d0);
            d0 = fmaf(qv[5], x1.y, d0);
            d0 = fmaf(qv[6], x1.z, d0);
            dot[u] = fmaf(qv[7], x1.w, d0);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
#pragma unroll
            for (int m = 1; m < LPC; m <<= 1) dot[u] += __shfl_xor(dot[u], m, kWave);
            const int j = j0 + u * CPI + grp;
            if (gl == 0 && j < n_cand) {
                float key = dot[u];          // ranked by the unscaled dot without the prior
                if (lambda) {
                    const int64_t c = cell_of[bh * M + slot[u]];
                    const float delta = (float)(i - c * cell) - 0.5f * (float)cell;
                    key = fmaf(dot[u], inv_sqrt_d,
                               lambda[h] * amax[bh * M + slot[u]] * erff(delta / (2.f * sigma[h])));
                }
                s_key[j] = float_key(key);
            }
        }
    }
    __syncthreads();
    if (!active || tq >= kWave) return;     // the query's first wavefront ranks
    const long orow = (bh * nq + row) * (long)topk;
    const float scale = lambda ? 1.f : inv_sqrt_d;
    // one search writes the slots (for the readout), the cells and the scores
    row_topk_write(
        s_key, n_cand, topk, lane,
        [&](int pos, int j, uint32_t kj) {
            const int sl = s_cand[j];
            idx_slot[orow + pos] = sl;
            if (idx_cell) idx_cell[orow + pos] = cell_of[bh * M + sl];
            if (score) score[orow + pos] = key_to_float(kj) * scale;
        },
        [&](int t) {
            idx_slot[orow + t] = -1;
            if (idx_cell) idx_cell[orow + t] = -1;
            if (score) score[orow + t] = 0.f;
        });
}

hipError_t launch_stream_select(int B, int H, int d, bool bf16, const void* q, const int64_t* qs,
                                const float* kbar, const float* amax, const int32_t* cell_of,
                                int M, const float* lambda, const float* sigma, int nq,
                                int64_t q_pos0, int window, int cell, const int32_t* keep,
                                const int32_t* keep_count, int keep_w, int64_t n_row0,
                                int rows_per_head, int topk, int32_t* idx_slot, int32_t* idx_cell,
                                float* score, hipStream_t st)
{
    if (nq == 0) return hipSuccess;
    // few queries (a decode step): the whole workgroup on one query
    const int qpb = nq * B * H < 1024 ? 1 : 4;
    const size_t lds = (size_t)2 * qpb * keep_w * sizeof(uint32_t);   // keys and the keep row
    if (lds > 65536) return hipErrorInvalidValue;
    const float inv_sqrt_d = 1.0f / sqrtf((float)d);
    dim3 grid((unsigned)((nq + qpb - 1) / qpb), (unsigned)(B * H)), block(256);
#define FS_STREAM_SELECT(E, D, QPB)                                                            \
    hipLaunchKernelGGL((stream_select_kernel<E, D, QPB>), grid, block, lds, st,                \
                       (const typename E::storage*)q, qs[0], qs[1], qs[2], kbar, amax, cell_of, \
                       M, lambda, sigma, H, nq, q_pos0, window, cell, keep, keep_count, keep_w, \
                       n_row0, rows_per_head, topk, inv_sqrt_d, idx_slot, idx_cell, score)
#define FS_STREAM_SELECT_Q(E, D) \
    if (qpb == 1) { FS_STREAM_SELECT(E, D, 1); } else { FS_STREAM_SELECT(E, D, 4); }
    if (bf16) {
        if (d == 64) { FS_STREAM_SELECT_Q(Bf16, 64) } else { FS_STREAM_SELECT_Q(Bf16, 128) }
    } else {
        if (d == 64) { FS_STREAM_SELECT_Q(F32, 64) } else { FS_STREAM_SELECT_Q(F32, 128) }
    }
#undef FS_STREAM_SELECT_Q
#undef FS_STREAM_SELECT
    return hipGetLastError();
}

namespace {

constexpr int kSelChunk = 32;        // union cells staged per chunk (two 16-cell MFMA blocks)
constexpr int kSelMaxCells = 32768;
constexpr int kSelMaxBlocks = 33;    // 16-cell score blocks per query: union of at most 528 cells

struct SelLayout {
    int nwords, u_cap, keep_w;
    size_t off_bitmap, off_rank, off_ulist, off_vmask, off_krows, bytes;
};

// LDS carve-up: kbar chunk split in 3 bf16 parts (swizzled rows), or two
// 64-key K tiles when reranking | bitmap | rank | union list | row-membership
// masks | copy of the keep rows.
template <int D>
__host__ __device__ inline SelLayout sel_layout(int n_hi, int u_cap, int keep_w, bool two_tiles = false,
                                                int rows = 3)
{
    SelLayout L;
    L.nwords = (n_hi + 31) / 32;
    L.u_cap = u_cap;
    L.keep_w = keep_w;
    auto up16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
    const size_t chunk = (size_t)3 * kSelChunk * D * 2, tiles = (size_t)2 * mf::kTileK * D * 2;
    size_t off = two_tiles && tiles > chunk ? tiles : chunk;
    L.off_bitmap = off;
    off = up16(off + (size_t)L.nwords * 4);
    L.off_rank = off;
    off = up16(off + (size_t)L.nwords * 2);
    L.off_ulist = off;
    off = up16(off + (size_t)u_cap * 2);
    L.off_vmask = off;
    off = up16(off + (size_t)u_cap * 4);
    L.off_krows = off;
    off = up16(off + (size_t)rows * keep_w * 2);
    L.bytes = off;
    return L;
}

__device__ __forceinline__ int sel_block_excl_scan(int x, int* red, int* total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
    }
    if (lane == kWave - 1) red[wv] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < nw; ++i) {
        before += i < wv ? red[i] : 0;
        all += red[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

// The four lanes n, n+16, n+32, n+48 of the MFMA output layout hold one query's
// scores.  Reductions over them use the gfx950 row swaps: after a swap with
// itself, the two results of a lane are its own value and its partner's.
template <class Op>
__device__ __forceinline__ uint32_t x4_reduce(uint32_t x, Op op)
{
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = op(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return op(b[0], b[1]);
}

// Exclusive prefix over g (lane n + 16 g, in g order) and total of packed
// counters: 5-bit fields, every partial sum below 32, so no field carries.
__device__ __forceinline__ void x4_scan(uint32_t v, int g, uint32_t& excl, uint32_t& total)
{
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const uint32_t p = a[0] + a[1] - v;                // row g ^ 1
    const uint32_t pair = v + p;
    const uint32_t s1 = (g & 1) ? pair : v;            // inclusive within the row pair
    const auto b = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
    const uint32_t other = b[0] + b[1] - pair;         // the other row pair's total
    excl = ((g & 2) ? s1 + other : s1) - v;
    total = pair + other;
}

constexpr int kFieldsPerWord = 6;   // 5-bit fields

__device__ __forceinline__ int field5(const uint32_t* w, int i)
{
    return (int)((w[i / kFieldsPerWord] >> (5 * (i % kFieldsPerWord))) & 31u);
}

}  // namespace

// Union of the candidate sets of a workgroup's queries (candidate counts n_a ..
// n_b): the keep rows copied to LDS, a bitmap over cells, per-word ranks, the
// union list ulist (slot -> cell) and vmask (bit r: the slot is in keep row
// n_a + r).  Without pruning the union is the prefix [0, n_b) and slot == cell.
// Returns the union size; ends with the block synchronised.
template <int ROWS>
__device__ __forceinline__ int sel_union(const int32_t* __restrict__ keep,
                                         const int32_t* __restrict__ keep_count, int keep_w,
                                         long bh, int n_lo, int n_rows, int n_a, int n_b,
                                         uint16_t* krows, uint32_t* bitmap, uint16_t* rank,
                                         uint16_t* ulist, uint32_t* vmask, int* red)
{
    const int tid = threadIdx.x;
    int n_union;
    if (keep != nullptr) {
        const int nw = (n_b + 31) >> 5;
        // the (at most ROWS) keep rows, copied to LDS with all loads in flight together
        const int r_first = n_a > 1 ? n_a : 1;            // rows of n = 0 are empty
        const int n_kr = n_b >= r_first ? n_b - r_first + 1 : 0;
        int kcnt[ROWS];
#pragma unroll
        for (int j = 0; j < ROWS; ++j)
            kcnt[j] = j < n_kr ? keep_count[bh * n_rows + (r_first + j - n_lo)] : 0;
        for (int e0 = 0; e0 < ROWS * keep_w; e0 += 4 * 256) {
            int vals[4];
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
                const int e = e0 + u4 * 256 + tid;
                const int j = e / keep_w, x = e - j * keep_w;
                int cnt = 0;
#pragma unroll
                for (int jj = 0; jj < ROWS; ++jj) cnt = j == jj ? kcnt[jj] : cnt;
                vals[u4] = (j < ROWS && x < cnt)
                               ? keep[(bh * n_rows + (r_first + j - n_lo)) * keep_w + x] : -1;
            }
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
                const int e = e0 + u4 * 256 + tid;
                if (e < ROWS * keep_w) krows[e] = (uint16_t)(vals[u4] < 0 ? 0xFFFF : vals[u4]);
            }
        }
        for (int wd = tid; wd < nw; wd += 256) bitmap[wd] = 0u;
        __syncthreads();
        for (int e = tid; e < ROWS * keep_w; e += 256) {
            const int c = krows[e];
            if (c != 0xFFFF) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
        }
        __syncthreads();
        const int wpt = (nw + 255) / 256;   // bitmap words per thread
        int mine = 0;
        for (int j = 0; j < wpt; ++j) {
            const int wd = tid * wpt + j;
            mine += wd < nw ? __popc(bitmap[wd]) : 0;
        }
        int run = sel_block_excl_scan(mine, red, &n_union);
        for (int j = 0; j < wpt; ++j) {
            const int wd = tid * wpt + j;
            if (wd < nw) {
                rank[wd] = (uint16_t)run;
                run += __popc(bitmap[wd]);
            }
        }
        __syncthreads();
        for (int wd = tid; wd < nw; wd += 256) {
            uint32_t bits = bitmap[wd];
            int r = rank[wd];
            while (bits) {
                const int bp = __ffs(bits) - 1;
                ulist[r] = (uint16_t)(32 * wd + bp);
                vmask[r] = 0u;
                ++r;
                bits &= bits - 1;
            }
        }
        __syncthreads();
        for (int e = tid; e < ROWS * keep_w; e += 256) {
            const int c = krows[e];
            if (c != 0xFFFF) {
                const int sl = rank[c >> 5] + __popc(bitmap[c >> 5] & ((1u << (c & 31)) - 1u));
                atomicOr(&vmask[sl], 1u << (r_first + e / keep_w - n_a));
            }
        }
    } else {
        n_union = n_b;   // candidates are the prefix [0, n_i); slot == cell
    }

    __syncthreads();                         // ulist / vmask complete
    return n_union;
}

// Exact top-K of each query over its four lanes (n, n+16, n+32, n+48), from the
// keys kv[bb][r] of union slots 16 bb + 4 g + r (0 = not a candidate), and the
// chosen cells written ascending to the query's idx row (score: the key's value
// times emit_scale).
template <int NB>
__device__ __forceinline__ void sel_topk_emit(const uint32_t (&kv)[NB][4], int topk, bool q_ok,
                                              int32_t* __restrict__ out_i, float* __restrict__ out_s,
                                              const int32_t* __restrict__ keep,
                                              const uint16_t* ulist, float emit_scale,
                                              int slot_base = 0)
{
    constexpr int kNW = (NB + kFieldsPerWord - 1) / kFieldsPerWord;
    constexpr int kKW = (4 * NB + 31) / 32;                    // kept-key mask words
    const int g = (threadIdx.x & 63) >> 4;
    int nv = 0;
    uint32_t k_and = 0xFFFFFFFFu, k_or = 0u;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t k = kv[bb][r];
            nv += k != 0u;
            k_and &= k != 0u ? k : 0xFFFFFFFFu;
            k_or |= k;
        }
    nv = (int)x4_reduce((uint32_t)nv, [](uint32_t x, uint32_t y) { return x + y; });
    k_and = x4_reduce(k_and, [](uint32_t x, uint32_t y) { return x & y; });
    k_or = x4_reduce(k_or, [](uint32_t x, uint32_t y) { return x | y; });
    const int kq = nv < topk ? nv : topk;
    // The kq-th largest key thr: the largest value with #{key >= thr} >= kq.
    // Bits above the highest bit in which two valid keys differ are common to
    // all of them and fixed from the start; the search stops for a query as soon
    // as exactly kq keys are >= the candidate (that set is then the top kq).
    const uint32_t diff = k_and ^ k_or;
    const int hb = diff != 0u ? 31 - __clz(diff) : -1;
    uint32_t thr = hb < 0 ? k_or : (k_or & ~(hb >= 31 ? 0xFFFFFFFFu : (2u << hb) - 1u));
    bool done = kq == 0 || hb < 0;
    int hb_w = done ? -1 : hb;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) hb_w = max(hb_w, __shfl_xor(hb_w, m, kWave));
    for (int bit = hb_w; bit >= 0; --bit) {
        if (__ballot(!done) == 0) break;
        const uint32_t cand = thr | (1u << bit);
        int c0 = 0, c1 = 0;                       // two chains: shorter dependency
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            c0 += (kv[bb][0] >= cand) + (kv[bb][1] >= cand);
            c1 += (kv[bb][2] >= cand) + (kv[bb][3] >= cand);
        }
        const int c = (int)x4_reduce((uint32_t)(c0 + c1), [](uint32_t x, uint32_t y) { return x + y; });
        if (!done && c >= kq) {
            thr = cand;
            done = c == kq;
        }
    }
    // thr >= 1 whenever kq > 0, so "key >= thr" and "key > thr" imply a valid key
    int ge = 0, gt = 0;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ge += kv[bb][r] >= thr;
            gt += kv[bb][r] > thr;
        }
    const int n_gt = (int)x4_reduce((uint32_t)gt, [](uint32_t x, uint32_t y) { return x + y; });
    const int n_ge = (int)x4_reduce((uint32_t)ge, [](uint32_t x, uint32_t y) { return x + y; });
    const int n_eq = n_ge - n_gt;
    const int need_eq = kq - n_gt;            // equal keys kept: those in the largest slots

    // kept keys as a bit mask over (bb, r)
    uint32_t km[kKW];
#pragma unroll
    for (int w = 0; w < kKW; ++w) km[w] = 0u;
    if (kq > 0) {
        uint32_t thr_o = thr;
        asm volatile("" : "+v"(thr_o));           // fresh compares below, not kept masks
        if (n_eq == need_eq) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kv[bb][r] >= thr_o) km[(4 * bb + r) / 32] |= 1u << ((4 * bb + r) % 32);
        } else {
            // ties at the threshold: rank the equal keys by slot, keep the top need_eq
            uint32_t cw[kNW], ex[kNW], tot[kNW];
#pragma unroll
            for (int w = 0; w < kNW; ++w) cw[w] = 0u;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                uint32_t e = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) e += kv[bb][r] == thr_o;
                cw[bb / kFieldsPerWord] += e << (5 * (bb % kFieldsPerWord));
            }
#pragma unroll
            for (int w = 0; w < kNW; ++w) x4_scan(cw[w], g, ex[w], tot[w]);
            int run = 0;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                int er = run + field5(ex, bb);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool is_eq = kv[bb][r] == thr_o;
                    const bool kept = kv[bb][r] > thr_o || (is_eq && er >= n_eq - need_eq);
                    er += is_eq;
                    if (kept) km[(4 * bb + r) / 32] |= 1u << ((4 * bb + r) % 32);
                }
                run += field5(tot, bb);
            }
        }
    }

    // ---- write the kept cells in ascending slot order -------------------------
    // Slot order is (bb, g, r): a kept key's position is the kept count of the
    // earlier blocks, of the lanes g' < g in its block, and of its own r' < r.
    {
        uint32_t cw[kNW], ex[kNW], tot[kNW];
#pragma unroll
        for (int w = 0; w < kNW; ++w) cw[w] = 0u;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            const uint32_t bits = (km[(4 * bb) / 32] >> ((4 * bb) % 32)) & 0xFu;
            cw[bb / kFieldsPerWord] += (uint32_t)__popc(bits) << (5 * (bb % kFieldsPerWord));
        }
#pragma unroll
        for (int w = 0; w < kNW; ++w) x4_scan(cw[w], g, ex[w], tot[w]);
        if (q_ok && kq > 0) {
            int run = 0;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                int p = run + field5(ex, bb);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if ((km[(4 * bb + r) / 32] >> ((4 * bb + r) % 32)) & 1u) {
                        const int slot = slot_base + 16 * bb + 4 * g + r;
                        out_i[p] = keep ? ulist[slot] : slot;
                        if (out_s) out_s[p] = key_to_float(kv[bb][r]) * emit_scale;
                        ++p;
                    }
                }
                run += field5(tot, bb);
            }
        }
    }
    if (q_ok) {
        for (int t = kq + g; t < topk; t += 4) {
            out_i[t] = -1;
            if (out_s) out_s[t] = 0.f;
        }
    }
}

// F32: fp32 storage.  q and kbar stay fp32 and the scores come from
// v_mfma_f32_16x16x4f32 (exact fp32 products, fp32 sums): lane group g supplies
// dimensions g*D/4 .. g*D/4 + D/4 - 1, so a lane keeps D/4 query floats and reads
// its cell row's D/4 consecutive floats from a padded fp32 chunk.
template <int D, int NB, bool F32 = false>
__global__ __launch_bounds__(256, (NB >= 33 || F32) ? 2 : 4) void select_topk_mfma_kernel(   // 256 threads exactly
    const void* __restrict__ qv, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ kbar, Prior pr, int H, int BH, int C, int nq, int q_pos0,
    int window, int cell, const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_count,
    int keep_w, int n_lo, int n_rows, int topk, int n_hi_all, int u_cap, float inv_sqrt_d,
    int32_t* __restrict__ idx, float* __restrict__ score, int n_split,
    int32_t* __restrict__ ws_cell, float* __restrict__ ws_val)
{
    using namespace mf;
    constexpr int KS = D / 32;
    constexpr int kTq = 64;                                    // queries per workgroup
    extern __shared__ uint4 smem_raw[];
    const SelLayout L = sel_layout<D>(n_hi_all, u_cap, keep ? keep_w : 0);
    char* base = reinterpret_cast<char*>(smem_raw);
    uint16_t* kbs = reinterpret_cast<uint16_t*>(base);      // [3 * kSelChunk] swizzled rows of D
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.off_bitmap);
    uint16_t* rank = reinterpret_cast<uint16_t*>(base + L.off_rank);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(base + L.off_ulist);
    uint32_t* vmask = reinterpret_cast<uint32_t*>(base + L.off_vmask);
    uint16_t* krows = reinterpret_cast<uint16_t*>(base + L.off_krows);
    __shared__ int red[4];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int h = (int)(bh % H), b = (int)(bh / H);
    // split `split` of n_split scores union slots s_base .. s_base + 16 NB - 1
    const int split = (int)(tb.tile % n_split);
    const long t0 = (tb.tile / n_split) * kTq;
    const int s_base = split * 16 * NB;
    const int n_rows_blk = nq - t0 < kTq ? (int)(nq - t0) : kTq;
    const int n_a = n_candidates((long)q_pos0 + t0, window, cell, C);
    const int n_b = n_candidates((long)q_pos0 + t0 + n_rows_blk - 1, window, cell, C);

    const int n_union = sel_union<3>(keep, keep_count, keep_w, bh, n_lo, n_rows, n_a, n_b, krows,
                                  bitmap, rank, ulist, vmask, red);

    // ---- the wave's 16 queries as B operands --------------------------------
    const int qr = 16 * wv + n;                 // this lane's query row in the block
    const bool q_ok = qr < n_rows_blk;
    const int n_q = q_ok ? n_candidates((long)q_pos0 + t0 + qr, window, cell, C) : 0;
    constexpr int T32 = D / 4, P32 = D + 4;     // fp32: dims per lane group, chunk row pitch
    bf16x8 qf[F32 ? 1 : KS];
    float qf32[F32 ? T32 : 1];
    if constexpr (F32) {
        const float* qrow = static_cast<const float*>(qv) + b * qs0 + h * qs1 +
                            (t0 + (q_ok ? qr : 0)) * qs2 + g * T32;
#pragma unroll
        for (int c = 0; c < T32 / 4; ++c) {
            const f32x4 x = q_ok ? *reinterpret_cast<const f32x4*>(qrow + 4 * c)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) qf32[4 * c + e] = x[e];
        }
    } else {
        const uint16_t* qrow = static_cast<const uint16_t*>(qv) + b * qs0 + h * qs1 +
                               (t0 + (q_ok ? qr : 0)) * qs2;
#pragma unroll
        for (int t = 0; t < KS; ++t)
            qf[t] = as_bf16x8(q_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * g)
                                   : make_uint4(0, 0, 0, 0));
    }

    // ---- scores S^T = Kbar Q^T over the union, kept in registers ------------
    // kv[bb][r] is the key of union slot 16 bb + 4 g + r for query n (0 when that
    // slot is not one of the query's candidates).  The next chunk's kbar rows are
    // loaded into registers while the current chunk's MFMAs run.
    constexpr int kIt = kSelChunk * D / 4 / 256;     // float4 per thread per chunk
    const float* kb_head = kbar + bh * (long)C * D;
    float4 pre[kIt];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int f = tid + 256 * it;
            const int cl = f / (D / 4), d4 = (f % (D / 4)) * 4;
            const int slot = c0 + cl;
            pre[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (slot < n_union) {
                const int c = keep ? ulist[slot] : slot;
                pre[it] = *reinterpret_cast<const float4*>(kb_head + (long)c * D + d4);
            }
        }
    };
    uint32_t kv[NB][4];
    load_chunk(s_base);
#pragma unroll
    for (int ci = 0; ci < (NB + 1) / 2; ++ci) {
        const int c0 = s_base + ci * kSelChunk;
        if (c0 < n_union) {                  // block-uniform
            __syncthreads();                 // previous chunk's MFMA reads are done
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int f = tid + 256 * it;
                const int cl = f / (D / 4), d4 = (f % (D / 4)) * 4;
                if constexpr (F32) {         // the fp32 row as it is, in a padded row
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(kbs) + cl * P32 + d4) =
                        f32x4{pre[it].x, pre[it].y, pre[it].z, pre[it].w};
                    continue;
                }
                const float r[4] = {pre[it].x, pre[it].y, pre[it].z, pre[it].w};
                // x = hi + mid + lo exactly: each residual has at most 16 (then 8)
                // significant bits, so the fp32 subtractions are exact.
                uint32_t part[3][2];
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    float a0 = r[e], a1 = r[e + 1];
                    const uint32_t hi = cvt_pk_bf16(a0, a1);
                    a0 -= __uint_as_float(hi << 16);
                    a1 -= __uint_as_float(hi & 0xFFFF0000u);
                    const uint32_t mid = cvt_pk_bf16(a0, a1);
                    a0 -= __uint_as_float(mid << 16);
                    a1 -= __uint_as_float(mid & 0xFFFF0000u);
                    part[0][e / 2] = hi;
                    part[1][e / 2] = mid;
                    part[2][e / 2] = cvt_pk_bf16(a0, a1);
                }
#pragma unroll
                for (int pp = 0; pp < 3; ++pp)
                    *reinterpret_cast<uint2*>(kbs + sw_off<D>(pp * kSelChunk + cl, d4 >> 3) + (d4 & 4)) =
                        make_uint2(part[pp][0], part[pp][1]);
            }
            __syncthreads();
            if (c0 + kSelChunk < n_union) load_chunk(c0 + kSelChunk);
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int bb = 2 * ci + b2;
                if (bb >= NB) break;
                const int slot0 = s_base + 16 * bb;
                if (slot0 < n_union) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (F32) {
                        const float* krow =
                            reinterpret_cast<const float*>(kbs) + (16 * b2 + n) * P32 + g * T32;
#pragma unroll
                        for (int c = 0; c < T32 / 4; ++c) {
                            const f32x4 a = *reinterpret_cast<const f32x4*>(krow + 4 * c);
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], qf32[4 * c + e], acc);
                        }
                    } else {
#pragma unroll
                        for (int t = 0; t < KS; ++t) {
#pragma unroll
                            for (int pp = 0; pp < 3; ++pp) {
                                const bf16x8 a = as_bf16x8(lds_load16(
                                    kbs + sw_off<D>(pp * kSelChunk + 16 * b2 + n, 4 * t + g)));
                                acc = mfma(a, qf[t], acc);
                            }
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int slot = slot0 + 4 * g + r;
                        bool ok = slot < n_union && n_q > 0;
                        if (ok) ok = keep ? ((vmask[slot] >> (n_q - n_a)) & 1u) != 0u : slot < n_q;
                        float rr = acc[r];   // the unscaled dot ranks alike without the prior
                        if (pr.lambda && ok)
                            rr = fmaf(rr, inv_sqrt_d,
                                      prior_term(pr, bh, h, C, (long)q_pos0 + t0 + qr,
                                                 keep ? ulist[slot] : slot, cell));
                        kv[bb][r] = ok ? float_key(rr) : 0u;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) kv[bb][r] = 0u;
                }
            }
        } else {
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int bb = 2 * ci + b2;
                if (bb < NB) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) kv[bb][r] = 0u;
                }
            }
        }
    }

    // ---- per query: exact top-K over its four lanes -------------------------
    const long orow = bh * nq + t0 + (q_ok ? qr : 0);
    if (n_split > 1) {         // this split's top K, with the exact key values, for the merge
        const long wrow = (orow * n_split + split) * (long)topk;
        sel_topk_emit<NB>(kv, topk, q_ok, ws_cell + wrow, ws_val + wrow, keep, ulist, 1.f,
                          s_base);
        return;
    }
    sel_topk_emit<NB>(kv, topk, q_ok, idx + orow * topk, score ? score + orow * topk : nullptr,
                      keep, ulist, pr.lambda ? 1.f : inv_sqrt_d);
}

// Merge of a split selection: per query, the n_split partial top-K lists (cells
// ascending within a split, splits in ascending slot order, so their valid
// entries concatenate to an ascending list) ranked again by the same keys.  One
// wavefront per query, four queries per workgroup.
__global__ __launch_bounds__(256) void select_merge_kernel(
    const int32_t* __restrict__ ws_cell, const float* __restrict__ ws_val, long rows, int n_split,
    int topk, float out_scale, int32_t* __restrict__ idx, float* __restrict__ score)
{
    extern __shared__ uint32_t smem[];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + wv;
    const int cap = n_split * topk;
    uint32_t* s_key = smem + wv * 2 * cap;
    int32_t* s_cell = reinterpret_cast<int32_t*>(s_key + cap);
    if (row >= rows) return;                        // no barrier below: whole waves leave
    const int32_t* wc = ws_cell + row * cap;
    const float* wk = ws_val + row * cap;
    // compact the valid entries (a prefix of each split's list, topk <= 64), in
    // split order; LDS accesses of one wavefront stay in order
    int n_valid = 0;
    for (int sp = 0; sp < n_split; ++sp) {
        const bool ok = lane < topk && wc[sp * topk + lane] >= 0;
        if (ok) {
            s_cell[n_valid + lane] = wc[sp * topk + lane];
            s_key[n_valid + lane] = float_key(wk[sp * topk + lane]);
        }
        n_valid += __popcll(__ballot(ok));
    }
    int32_t* out_i = idx + row * topk;
    float* out_s = score ? score + row * topk : nullptr;
    row_topk_write(
        s_key, n_valid, topk, lane,
        [&](int pos, int j, uint32_t kj) {
            out_i[pos] = s_cell[j];
            if (out_s) out_s[pos] = key_to_float(kj) * out_scale;
        },
        [&](int t) {
            out_i[t] = -1;
            if (out_s) out_s[t] = 0.f;
        });
}

// Combine two partial log-sum-exps (m: max logit in log2 units, z: sum of
// exp2(logit - m), z >= 1) into one; one exp2, and symmetric in its operands
// only through their order, which both lanes of a pair share.
__device__ __forceinline__ void lse_merge(float ma, float za, float mb, float zb, float& m,
                                          float& z)
{
    const float dlt = mb - ma;
    const float e = __builtin_amdgcn_exp2f(-fabsf(dlt));
    m = __builtin_elementwise_maximum(ma, mb);
    z = dlt <= 0.f ? fmaf(zb, e, za) : fmaf(za, e, zb);
}

// Token-level reranking (section 3.4, eq. 12) and top-K.  The same workgroup
// shape, candidate union and selection as the kernel above; the score of union
// slot u for query n is the log-sum-exp of the s = 32 logits q.k_j / sqrt(d) of
// its cell's tokens (+ the eq. 7 prior).  Tiles of two cells (64 keys) are staged
// in LDS (swizzled, bf16 as stored; two buffers, one barrier per tile) and
// multiplied by the wave's 16 queries on the matrix core.  A cell's 32 logits of
// a query sit in the query's four lanes (8 each): each lane reduces its 8 to a
// partial (max, sum of exp2), one lane-half swap merges the partials of both
// cells at once (lanes 0-31 then hold the first cell, 32-63 the second) and a
// row swap finishes them.  Tile t of 16-slot block bb holds slots 16 bb + t and
// 16 bb + 8 + t, so each result lands in the lane that keeps its slot.  Tile
// u + 2 is loaded into registers while tile u is scored and tile u + 1 is
// written to the other buffer.
template <int D, int NB>
__global__ __launch_bounds__(256, NB >= 33 ? 1 : (NB >= 17 ? 3 : 4)) void rerank_topk_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const uint16_t* __restrict__ k, int64_t kvs0, int64_t kvs1, int64_t kvs2, Prior pr, int H,
    int BH, int C, int nq, int q_pos0, int window, int cell, const int32_t* __restrict__ keep,
    const int32_t* __restrict__ keep_count, int keep_w, int n_lo, int n_rows, int topk,
    int n_hi_all, int u_cap, float inv_sqrt_d, int32_t* __restrict__ idx,
    float* __restrict__ score)
{
    using namespace mf;
    constexpr int KS = D / 32;
    constexpr int kTq = 64;
    constexpr int KC = (kTileK * D / 8) / 256;            // 16-byte K chunks per thread
    extern __shared__ uint4 smem_raw[];
    const SelLayout L = sel_layout<D>(n_hi_all, u_cap, keep ? keep_w : 0, true);
    char* base = reinterpret_cast<char*>(smem_raw);
    uint16_t* ks = reinterpret_cast<uint16_t*>(base);       // two swizzled 64-key tiles
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.off_bitmap);
    uint16_t* rank = reinterpret_cast<uint16_t*>(base + L.off_rank);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(base + L.off_ulist);
    uint32_t* vmask = reinterpret_cast<uint32_t*>(base + L.off_vmask);
    uint16_t* krows = reinterpret_cast<uint16_t*>(base + L.off_krows);
    __shared__ int red[4];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const long t0 = tb.tile * kTq;
    const int n_rows_blk = nq - t0 < kTq ? (int)(nq - t0) : kTq;
    const int n_a = n_candidates((long)q_pos0 + t0, window, cell, C);
    const int n_b = n_candidates((long)q_pos0 + t0 + n_rows_blk - 1, window, cell, C);
    const int n_union = sel_union<3>(keep, keep_count, keep_w, bh, n_lo, n_rows, n_a, n_b, krows,
                                  bitmap, rank, ulist, vmask, red);

    const int qr = 16 * wv + n;
    const bool q_ok = qr < n_rows_blk;
    const long qpos = (long)q_pos0 + t0 + qr;
    const int n_q = q_ok ? n_candidates(qpos, window, cell, C) : 0;
    bf16x8 qf[KS];
    {
        const uint16_t* qrow = q + b * qs0 + h * qs1 + (t0 + (q_ok ? qr : 0)) * qs2;
#pragma unroll
        for (int t = 0; t < KS; ++t)
            qf[t] = as_bf16x8(q_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * g)
                                   : make_uint4(0, 0, 0, 0));
    }

    // Tile u (block bb = u / 8, t = u % 8) holds union slots 16 bb + t and
    // 16 bb + 8 + t; a second slot past the union repeats the first cell (its
    // score is masked below).  The tile count covers every slot below n_union.
    const uint16_t* kh = k + b * kvs0 + h * kvs1;
    uint32_t koff[KC];                                  // byte offset of this thread's chunks in a cell
#pragma unroll
    for (int it = 0; it < KC; ++it) {
        const int cidx = tid + 256 * it;
        koff[it] = (uint32_t)((((cidx / (D / 8)) & 31) * kvs2 + (cidx % (D / 8)) * 8) * 2);
    }
    uint4 st[KC];
    auto load_tile = [&](int u) {
        const int s0 = 16 * (u >> 3) + (u & 7);
        const int s1 = s0 + 8 < n_union ? s0 + 8 : s0;
        const int c0 = __builtin_amdgcn_readfirstlane(keep ? (int)ulist[s0] : s0);
        const int c1 = __builtin_amdgcn_readfirstlane(keep ? (int)ulist[s1] : s1);
        const char* p0 = reinterpret_cast<const char*>(kh + (long)c0 * cell * kvs2);
        const char* p1 = reinterpret_cast<const char*>(kh + (long)c1 * cell * kvs2);
#pragma unroll
        for (int it = 0; it < KC; ++it)      // rows 0-31 of the tile: first cell
            st[it] = *reinterpret_cast<const uint4*>((it < KC / 2 ? p0 : p1) + koff[it]);
    };
    auto store_tile = [&](uint16_t* buf) {
#pragma unroll
        for (int it = 0; it < KC; ++it) {
            const int cidx = tid + 256 * it;
            lds_store16(buf + ksw_off<D>(cidx / (D / 8), cidx % (D / 8)), st[it]);
        }
    };
    const int n_full = n_union >> 4, rem = n_union & 15;
    const int n_tiles = 8 * n_full + (rem < 8 ? rem : 8);
    const float scale_log2 = inv_sqrt_d * 1.4426950408889634f;
    // kv[bb][r]: the log-sum-exp of union slot 16 bb + 4 g + r (float bits) until
    // the loop ends, then its selection key
    uint32_t kv[NB][4];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) kv[bb][r] = 0u;
    float v[4] = {0.f, 0.f, 0.f, 0.f};             // the current 16-slot block's values
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(ks);
        if (n_tiles > 1) load_tile(1);
    }
    for (int u = 0; u < n_tiles; ++u) {
        __syncthreads();        // tile u is in buffer u % 2; reads of tile u - 1 are done
        if (u + 1 < n_tiles) {
            store_tile(ks + ((u + 1) & 1) * (kTileK * D));
            if (u + 2 < n_tiles) load_tile(u + 2);
        }
        const uint16_t* kt = ks + (u & 1) * (kTileK * D);
        f32x4 s4[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s4[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < KS; ++tt)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                s4[kb] = mfma(as_bf16x8(lds_load16(kt + ksw_off<D>(16 * kb + n, 4 * tt + g))),
                              qf[tt], s4[kb]);
        // this lane's partial (max, sum) of each cell: logits of keys 16 kb + 4 g + r
        float pm[2], pz[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            const f32x4 &x = s4[2 * c2], &y = s4[2 * c2 + 1];
            // IEEE maximum: MFMA results need no NaN quieting first (finite here)
            auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
            const float m = mx(mx(mx(x[0], x[1]), mx(x[2], x[3])), mx(mx(y[0], y[1]), mx(y[2], y[3])));
            const float mb = m * scale_log2;
            float z0 = __builtin_amdgcn_exp2f(fmaf(x[0], scale_log2, -mb));
            float z1 = __builtin_amdgcn_exp2f(fmaf(y[0], scale_log2, -mb));
#pragma unroll
            for (int r = 1; r < 4; ++r) {
                z0 += __builtin_amdgcn_exp2f(fmaf(x[r], scale_log2, -mb));
                z1 += __builtin_amdgcn_exp2f(fmaf(y[r], scale_log2, -mb));
            }
            pm[c2] = mb;
            pz[c2] = z0 + z1;
        }
        // lanes 0-31 pair up halves of the first cell, lanes 32-63 of the second
        const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[0]),
                                                         __float_as_uint(pm[1]), false, false);
        const auto sz = __builtin_amdgcn_permlane32_swap(__float_as_uint(pz[0]),
                                                         __float_as_uint(pz[1]), false, false);
        float m1, z1;
        lse_merge(__uint_as_float(sm[0]), __uint_as_float(sz[0]), __uint_as_float(sm[1]),
                  __uint_as_float(sz[1]), m1, z1);
        // then rows l and l ^ 16
        const auto tm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m1), __float_as_uint(m1),
                                                         false, false);
        const auto tz = __builtin_amdgcn_permlane16_swap(__float_as_uint(z1), __float_as_uint(z1),
                                                         false, false);
        float m2, z2;
        lse_merge(__uint_as_float(tm[0]), __uint_as_float(tz[0]), __uint_as_float(tm[1]),
                  __uint_as_float(tz[1]), m2, z2);
        const float lse = (m2 + __log2f(z2)) * 0.6931471805599453f;
        // slot 16 bb + 8 c2 + t is kept by lane row g = 2 c2 + t / 4 at r = t % 4
        const int t = u & 7;
        const bool mine = (g & 1) == (t >> 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = mine && r == (t & 3) ? lse : v[r];
        if (t == 7 || u + 1 == n_tiles) {          // block-uniform: the 16-slot block is done
            const int bbu = u >> 3;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
                if (bb == bbu) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) kv[bb][r] = __float_as_uint(v[r]);
                }
        }
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int slot = 16 * bb + 4 * g + r;
            bool ok = slot < n_union && n_q > 0;
            if (ok) ok = keep ? ((vmask[slot] >> (n_q - n_a)) & 1u) != 0u : slot < n_q;
            float rr = __uint_as_float(kv[bb][r]);
            if (pr.lambda && ok)
                rr += prior_term(pr, bh, h, C, qpos, keep ? ulist[slot] : slot, cell);
            kv[bb][r] = ok ? float_key(rr) : 0u;
        }

    const long orow = bh * nq + t0 + (q_ok ? qr : 0);
    sel_topk_emit<NB>(kv, topk, q_ok, idx + orow * topk, score ? score + orow * topk : nullptr,
                      keep, ulist, 1.f);
}

// Reranking (eq. 12) for 128 queries per workgroup on the 32x32x16 matrix core,
// when the caller gives a workspace.  A wave scores its 32 queries against each
// 32-key cell in one 32x32 block, so every K fragment read from LDS serves 32
// queries (twice the 16x16 kernel above), and a query's 32 logits of a cell sit
// in lanes l and l + 32 (16 each): a local (max, sum of exp2) per lane, then one
// lane-half swap merges both cells of the tile at once.  The per-slot scores go
// to the workspace, [workgroup][union slot][query], and are read back in two
// rounds of 16 queries for the same exact top-K search as the kernels above.
// The union spans at most five keep rows (128 consecutive queries).
template <int D, int NB>
__global__ __launch_bounds__(256, NB >= 33 ? 2 : 4) void rerank32_kernel(
    const uint16_t* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const uint16_t* __restrict__ k, int64_t kvs0, int64_t kvs1, int64_t kvs2, Prior pr, int H,
    int BH, int C, int nq, int q_pos0, int window, int cell, const int32_t* __restrict__ keep,
    const int32_t* __restrict__ keep_count, int keep_w, int n_lo, int n_rows, int topk,
    int n_hi_all, int u_cap, float inv_sqrt_d, float* __restrict__ ws,
    int32_t* __restrict__ idx, float* __restrict__ score)
{
    using namespace mf;
    constexpr int KS = D / 16;                              // k-steps of 32x32x16
    constexpr int kTq = 128;
    constexpr int KC = (kTileK * D / 8) / 256;              // 16-byte K chunks per thread
    extern __shared__ uint4 smem_raw[];
    const SelLayout L = sel_layout<D>(n_hi_all, u_cap, keep ? keep_w : 0, true, 5);
    char* base = reinterpret_cast<char*>(smem_raw);
    uint16_t* ks = reinterpret_cast<uint16_t*>(base);       // two swizzled 64-key tiles
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.off_bitmap);
    uint16_t* rank = reinterpret_cast<uint16_t*>(base + L.off_rank);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(base + L.off_ulist);
    uint32_t* vmask = reinterpret_cast<uint32_t*>(base + L.off_vmask);
    uint16_t* krows = reinterpret_cast<uint16_t*>(base + L.off_krows);
    __shared__ int red[4];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const long t0 = tb.tile * kTq;
    const int n_rows_blk = nq - t0 < kTq ? (int)(nq - t0) : kTq;
    const int n_a = n_candidates((long)q_pos0 + t0, window, cell, C);
    const int n_b = n_candidates((long)q_pos0 + t0 + n_rows_blk - 1, window, cell, C);
    const int n_union = sel_union<5>(keep, keep_count, keep_w, bh, n_lo, n_rows, n_a, n_b,
                                     krows, bitmap, rank, ulist, vmask, red);

    // the wave's 32 queries as B operands: lane l holds query 32 wv + l % 32,
    // dims 16 ks + 8 (l / 32) .. + 7
    const int qc = 32 * wv + (lane & 31);
    const bool qc_ok = qc < n_rows_blk;
    bf16x8 qf[KS];
    {
        const uint16_t* qrow = q + b * qs0 + h * qs1 + (t0 + (qc_ok ? qc : 0)) * qs2;
#pragma unroll
        for (int t = 0; t < KS; ++t)
            qf[t] = as_bf16x8(qc_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * t + 8 * (lane >> 5))
                                    : make_uint4(0, 0, 0, 0));
    }

    // tile u holds union slots 2u (rows 0-31) and 2u + 1 (rows 32-63; past the
    // union it repeats the first cell)
    const uint16_t* kh = k + b * kvs0 + h * kvs1;
    uint32_t koff[KC];
#pragma unroll
    for (int it = 0; it < KC; ++it) {
        const int cidx = tid + 256 * it;
        koff[it] = (uint32_t)((((cidx / (D / 8)) & 31) * kvs2 + (cidx % (D / 8)) * 8) * 2);
    }
    uint4 st[KC];
    auto load_tile = [&](int u) {
        const int s0 = 2 * u, s1 = 2 * u + 1 < n_union ? 2 * u + 1 : 2 * u;
        const int c0 = __builtin_amdgcn_readfirstlane(keep ? (int)ulist[s0] : s0);
        const int c1 = __builtin_amdgcn_readfirstlane(keep ? (int)ulist[s1] : s1);
        const char* p0 = reinterpret_cast<const char*>(kh + (long)c0 * cell * kvs2);
        const char* p1 = reinterpret_cast<const char*>(kh + (long)c1 * cell * kvs2);
#pragma unroll
        for (int it = 0; it < KC; ++it)
            st[it] = *reinterpret_cast<const uint4*>((it < KC / 2 ? p0 : p1) + koff[it]);
    };
    auto store_tile = [&](uint16_t* buf) {
#pragma unroll
        for (int it = 0; it < KC; ++it) {
            const int cidx = tid + 256 * it;
            lds_store16(buf + ksw_off<D>(cidx / (D / 8), cidx % (D / 8)), st[it]);
        }
    };
    const int n_tiles = (n_union + 1) / 2;
    const float scale_log2 = inv_sqrt_d * 1.4426950408889634f;
    float* wsb = ws + (long)blockIdx.x * ((u_cap + 15) & ~15) * kTq;   // [slot][query]
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(ks);
        if (n_tiles > 1) load_tile(1);
    }
    for (int u = 0; u < n_tiles; ++u) {
        __syncthreads();        // tile u is in buffer u % 2; reads of tile u - 1 are done
        if (u + 1 < n_tiles) {
            store_tile(ks + ((u + 1) & 1) * (kTileK * D));
            if (u + 2 < n_tiles) load_tile(u + 2);
        }
        const uint16_t* kt = ks + (u & 1) * (kTileK * D);
        f32x16 sc[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[c2][e] = 0.f;
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
                sc[c2] = mfma32(as_bf16x8(lds_load16(kt + ksw_off<D>(32 * c2 + (lane & 31),
                                                                     2 * t + (lane >> 5)))),
                                qf[t], sc[c2]);
        // this lane's partial (max, sum) of each cell: 16 of the query's 32 logits
        float pm[2], pz[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            auto mx = [](float a, float bb) { return __builtin_elementwise_maximum(a, bb); };
            float m = sc[c2][0];
#pragma unroll
            for (int e = 1; e < 16; ++e) m = mx(m, sc[c2][e]);
            const float mb = m * scale_log2;
            float z0 = __builtin_amdgcn_exp2f(fmaf(sc[c2][0], scale_log2, -mb));
            float z1 = __builtin_amdgcn_exp2f(fmaf(sc[c2][1], scale_log2, -mb));
#pragma unroll
            for (int e = 2; e < 16; e += 2) {
                z0 += __builtin_amdgcn_exp2f(fmaf(sc[c2][e], scale_log2, -mb));
                z1 += __builtin_amdgcn_exp2f(fmaf(sc[c2][e + 1], scale_log2, -mb));
            }
            pm[c2] = mb;
            pz[c2] = z0 + z1;
        }
        // lanes 0-31 pair up the halves of the first cell, lanes 32-63 of the second
        const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[0]),
                                                         __float_as_uint(pm[1]), false, false);
        const auto sz = __builtin_amdgcn_permlane32_swap(__float_as_uint(pz[0]),
                                                         __float_as_uint(pz[1]), false, false);
        float m1, z1;
        lse_merge(__uint_as_float(sm[0]), __uint_as_float(sz[0]), __uint_as_float(sm[1]),
                  __uint_as_float(sz[1]), m1, z1);
        const int slot = 2 * u + (lane >> 5);
        if (slot < n_union) wsb[slot * kTq + qc] = (m1 + __log2f(z1)) * 0.6931471805599453f;
    }
    __syncthreads();            // the scores are visible to the whole workgroup

    // ---- per query: exact top-K over its four lanes, 16 queries per round ----
    const int n = lane & 15, g = lane >> 4;
    for (int ro = 0; ro < 2; ++ro) {
        const int qr = 32 * wv + 16 * ro + n;
        const bool q_ok = qr < n_rows_blk;
        const long qpos = (long)q_pos0 + t0 + qr;
        const int n_q = q_ok ? n_candidates(qpos, window, cell, C) : 0;
        uint32_t kv[NB][4];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = 16 * bb + 4 * g + r;
                bool ok = slot < n_union && n_q > 0;
                if (ok) ok = keep ? ((vmask[slot] >> (n_q - n_a)) & 1u) != 0u : slot < n_q;
                float rr = ok ? wsb[slot * kTq + qr] : 0.f;
                if (pr.lambda && ok)
                    rr += prior_term(pr, bh, h, C, qpos, keep ? ulist[slot] : slot, cell);
                kv[bb][r] = ok ? float_key(rr) : 0u;
            }
        const long orow = bh * nq + t0 + (q_ok ? qr : 0);
        sel_topk_emit<NB>(kv, topk, q_ok, idx + orow * topk,
                          score ? score + orow * topk : nullptr, keep, ulist, 1.f);
    }
}

namespace {

// Top-K over the candidates of every query: eq. 7 scores from kbar, or (rerank)
// eq. 12 scores from the keys k.  MFMA kernels (selection for both storage
// types, reranking for bf16) when every query's candidates fit the register
// blocks; row-wise kernels otherwise.
// Largest candidate list: the keep width, or every cell below the last query's n.
int largest_candidate_count(const Shape& sh)
{
    int n_hi = 0;
    const long i = (long)sh.q_pos0 + sh.nq - 1;
    if (i >= sh.w) n_hi = (int)((i - sh.w) / sh.s);
    return n_hi > sh.C ? sh.C : n_hi;
}

// Union slots the 128-query reranking kernel provides for (at most five keep rows),
// in 16-slot blocks.
int rerank32_slots(const Shape& sh, bool pruned, int keep_w)
{
    const int n_hi = largest_candidate_count(sh);
    const int u_cap = pruned ? (keep_w + 5 < n_hi ? keep_w + 5 : n_hi) : n_hi;
    return ((u_cap > 0 ? u_cap : 1) + 15) & ~15;
}

// Union slots the 64-query selection kernel provides for (at most three keep
// rows), in 16-slot blocks.
int select_slots(const Shape& sh, bool pruned, int keep_w)
{
    const int n_hi = largest_candidate_count(sh);
    const int u_cap = pruned ? (keep_w + 3 < n_hi ? keep_w + 3 : n_hi) : n_hi;
    return ((u_cap > 0 ? u_cap : 1) + 15) & ~15;
}

hipError_t launch_topk(const Shape& sh, const void* q, const float* kbar, const void* k,
                       const Prior& pr, const int32_t* keep, const int32_t* keep_count,
                       int keep_w, int n_lo, int n_rows, int topk, int32_t* idx, float* score,
                       bool rerank, void* ws, size_t ws_bytes, hipStream_t st)
{
    if (sh.nq == 0) return hipSuccess;
    const int n_hi = largest_candidate_count(sh);
    const float inv_sqrt_d = 1.0f / sqrtf((float)sh.d);
    // reranking addresses a cell's rows with 32-bit byte offsets
    const bool offs_ok = !rerank || ((int64_t)(sh.s - 1) * sh.kvs[2] + sh.d) * 2 < (1ll << 31);
    if (rerank && ws && ws_bytes >= rerank_ws_bytes(sh, keep != nullptr, keep_w)) {
        const int uc = rerank32_slots(sh, keep != nullptr, keep_w);
        const int kw = keep ? keep_w : 0;
        const size_t lds = sh.d == 64 ? sel_layout<64>(n_hi, uc, kw, true, 5).bytes
                                      : sel_layout<128>(n_hi, uc, kw, true, 5).bytes;
        if (sh.bf16 && lds <= 64 * 1024 && sh.C <= kSelMaxCells && uc <= 16 * kSelMaxBlocks &&
            offs_ok) {
            dim3 grid((unsigned)((sh.nq + 127) / 128 * sh.B * sh.H));
            const int nb_need = uc / 16;
            note_path("rerank: MFMA, 128 queries per workgroup, scores in the workspace");
#define FS_RERANK32(D, NB)                                                                      \
            hipLaunchKernelGGL((rerank32_kernel<D, NB>), grid, dim3(256), lds, st,              \
                               (const uint16_t*)q, sh.qs[0], sh.qs[1], sh.qs[2],                 \
                               (const uint16_t*)k, sh.kvs[0], sh.kvs[1], sh.kvs[2], pr, sh.H,    \
                               sh.B * sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep,            \
                               keep_count, keep_w, n_lo, n_rows, topk, n_hi, uc, inv_sqrt_d,     \
                               static_cast<float*>(ws), idx, score)
#define FS_RERANK32_NB(D)                                                                       \
            if (nb_need <= 2) { FS_RERANK32(D, 2); }                                            \
            else if (nb_need <= 4) { FS_RERANK32(D, 4); }                                       \
            else if (nb_need <= 9) { FS_RERANK32(D, 9); }                                       \
            else if (nb_need <= 17) { FS_RERANK32(D, 17); }                                     \
            else { FS_RERANK32(D, 33); }
            if (sh.d == 64) { FS_RERANK32_NB(64) } else { FS_RERANK32_NB(128) }
#undef FS_RERANK32_NB
#undef FS_RERANK32
            return hipGetLastError();
        }
    }
    {
        const int u_cap = keep ? (keep_w + 3 < n_hi ? keep_w + 3 : n_hi) : n_hi;
        const int uc = ((u_cap > 0 ? u_cap : 1) + 15) & ~15;     // 16-cell blocks
        const int kw = keep ? keep_w : 0;
        const size_t lds = sh.d == 64 ? sel_layout<64>(n_hi, uc, kw, rerank).bytes
                                      : sel_layout<128>(n_hi, uc, kw, rerank).bytes;
        if ((sh.bf16 || !rerank) && lds <= 64 * 1024 && sh.C <= kSelMaxCells &&
            uc <= 16 * kSelMaxBlocks && offs_ok) {
            const bool f32 = !sh.bf16;
            // short query ranges: the union split over workgroups of 64 slots each,
            // then a merge of their top-K lists (selection with a workspace only)
            const int S = !rerank && ws && ws_bytes >= select_ws_bytes(sh, keep != nullptr, keep_w,
                                                                      topk)
                              ? select_splits(sh, keep != nullptr, keep_w) : 1;
            if (S > 1) {
                note_path("select: %sMFMA, union split over %d workgroups, then a merge",
                          f32 ? "fp32 " : "", S);
                int32_t* ws_cell = static_cast<int32_t*>(ws);
                float* ws_val = reinterpret_cast<float*>(ws_cell + (size_t)sh.B * sh.H * sh.nq * S * topk);
                dim3 grid_s((unsigned)((sh.nq + 63) / 64 * S * sh.B * sh.H));
#define FS_SELECT_SPLIT(D, F)                                                                   \
                hipLaunchKernelGGL((select_topk_mfma_kernel<D, 4, F>), grid_s, dim3(256), lds,  \
                                   st, q, sh.qs[0], sh.qs[1], sh.qs[2], kbar, pr, sh.H,          \
                                   sh.B * sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep,        \
                                   keep_count, keep_w, n_lo, n_rows, topk, n_hi, uc, inv_sqrt_d, \
                                   idx, score, S, ws_cell, ws_val)
                if (f32) {
                    if (sh.d == 64) { FS_SELECT_SPLIT(64, true); } else { FS_SELECT_SPLIT(128, true); }
                } else {
                    if (sh.d == 64) { FS_SELECT_SPLIT(64, false); } else { FS_SELECT_SPLIT(128, false); }
                }
#undef FS_SELECT_SPLIT
                hipError_t err = hipGetLastError();
                if (err != hipSuccess) return err;
                const long rows = (long)sh.B * sh.H * sh.nq;
                hipLaunchKernelGGL(select_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256),
                                   (size_t)4 * 2 * S * topk * sizeof(uint32_t), st, ws_cell, ws_val,
                                   rows, S, topk, pr.lambda ? 1.f : inv_sqrt_d, idx, score);
                return hipGetLastError();
            }
            dim3 grid((unsigned)((sh.nq + 63) / 64 * sh.B * sh.H));
            const int nb_need = uc / 16;
            note_path("%s: %sMFMA, 64 queries per workgroup", rerank ? "rerank" : "select",
                      f32 ? "fp32 " : "");
#define FS_SELECT_MFMA(D, NB)                                                                   \
            if (f32)                                                                            \
                hipLaunchKernelGGL((select_topk_mfma_kernel<D, NB, true>), grid, dim3(256), lds,\
                                   st, q, sh.qs[0], sh.qs[1], sh.qs[2], kbar, pr, sh.H,          \
                                   sh.B * sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep,        \
                                   keep_count, keep_w, n_lo, n_rows, topk, n_hi, uc, inv_sqrt_d, \
                                   idx, score, 1, nullptr, nullptr);                             \
            else if (rerank)                                                                    \
                hipLaunchKernelGGL((rerank_topk_mfma_kernel<D, NB>), grid, dim3(256), lds, st,  \
                                   (const uint16_t*)q, sh.qs[0], sh.qs[1], sh.qs[2],             \
                                   (const uint16_t*)k, sh.kvs[0], sh.kvs[1], sh.kvs[2], pr,      \
                                   sh.H, sh.B * sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep,  \
                                   keep_count, keep_w, n_lo, n_rows, topk, n_hi, uc, inv_sqrt_d, \
                                   idx, score);                                                  \
            else                                                                                \
                hipLaunchKernelGGL((select_topk_mfma_kernel<D, NB>), grid, dim3(256), lds, st,  \
                                   q, sh.qs[0], sh.qs[1], sh.qs[2], kbar, pr,                    \
                                   sh.H, sh.B * sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep,  \
                                   keep_count, keep_w, n_lo, n_rows, topk, n_hi, uc, inv_sqrt_d, \
                                   idx, score, 1, nullptr, nullptr)
#define FS_SELECT_NB(D)                                                                         \
            if (nb_need <= 2) { FS_SELECT_MFMA(D, 2); }                                         \
            else if (nb_need <= 4) { FS_SELECT_MFMA(D, 4); }                                    \
            else if (nb_need <= 9) { FS_SELECT_MFMA(D, 9); }                                    \
            else if (nb_need <= 17) { FS_SELECT_MFMA(D, 17); }                                  \
            else { FS_SELECT_MFMA(D, 33); }
            if (sh.d == 64) { FS_SELECT_NB(64) } else { FS_SELECT_NB(128) }
#undef FS_SELECT_NB
#undef FS_SELECT_MFMA
            return hipGetLastError();
        }
    }
    {
        const int u_cap = keep ? (keep_w + 3 < n_hi ? keep_w + 3 : n_hi) : n_hi;
        note_path("%s: row-wise, one wavefront per query (%s)", rerank ? "rerank" : "select",
                  !sh.bf16 && rerank ? "fp32 storage"
                  : sh.C > kSelMaxCells ? "more than 32768 cells"
                  : u_cap > 16 * kSelMaxBlocks ? "candidate union wider than 528 cells"
                  : "bookkeeping exceeds 64 KiB of LDS");
    }
    const int cap = keep ? keep_w : (n_hi > 0 ? n_hi : 1);
    // As many waves (query rows) per block as fit in 64 KiB of LDS.
    int waves = kSelWaves;
    while (waves > 1 && (size_t)waves * (sh.d + cap) * sizeof(uint32_t) > 65536) waves >>= 1;
    const size_t lds = (size_t)waves * (sh.d + cap) * sizeof(uint32_t);
    if (lds > 65536) return hipErrorInvalidValue;
    dim3 grid((unsigned)((sh.nq + waves - 1) / waves), (unsigned)(sh.B * sh.H));
    dim3 block(waves * kWave);
#define FS_SELECT(E, D, RR)                                                                    \
    hipLaunchKernelGGL((select_topk_kernel<E, D, RR>), grid, block, lds, st,                   \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2], kbar,       \
                       (const typename E::storage*)k, sh.kvs[0], sh.kvs[1], sh.kvs[2], pr,      \
                       sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep, keep_count, keep_w, n_lo,\
                       n_rows, topk, cap, inv_sqrt_d, idx, score)
#define FS_SELECT_RR(E, D)                                                                     \
    if (rerank) { FS_SELECT(E, D, true); } else { FS_SELECT(E, D, false); }
    if (sh.bf16) {
        if (sh.d == 64) { FS_SELECT_RR(Bf16, 64) } else { FS_SELECT_RR(Bf16, 128) }
    } else {
        if (sh.d == 64) { FS_SELECT_RR(F32, 64) } else { FS_SELECT_RR(F32, 128) }
    }
#undef FS_SELECT_RR
#undef FS_SELECT
    return hipGetLastError();
}

}  // namespace

int select_splits(const Shape& sh, bool pruned, int keep_w)
{
    const long blocks = (long)(sh.nq + 63) / 64 * sh.B * sh.H;
    const int uc = select_slots(sh, pruned, keep_w);
    if (blocks >= 256 || uc <= 64 || uc > 16 * kSelMaxBlocks) return 1;
    return (uc + 63) / 64;            // 64 slots (four 16-slot blocks) per split
}

size_t select_ws_bytes(const Shape& sh, bool pruned, int keep_w, int topk)
{
    const int S = select_splits(sh, pruned, keep_w);
    if (S <= 1) return 0;
    return (size_t)sh.B * sh.H * sh.nq * S * topk * (sizeof(int32_t) + sizeof(float));
}

hipError_t launch_select(const Shape& sh, const void* q, const float* kbar, const Prior& pr,
                         const int32_t* keep, const int32_t* keep_count, int keep_w, int n_lo,
                         int n_rows, int topk, int32_t* idx, float* score, void* ws,
                         size_t ws_bytes, hipStream_t st)
{
    return launch_topk(sh, q, kbar, nullptr, pr, keep, keep_count, keep_w, n_lo, n_rows, topk,
                       idx, score, false, ws, ws_bytes, st);
}

size_t rerank_ws_bytes(const Shape& sh, bool pruned, int keep_w)
{
    const size_t blocks = (size_t)(sh.nq + 127) / 128 * sh.B * sh.H;
    return blocks * rerank32_slots(sh, pruned, keep_w) * 128 * sizeof(float);
}

hipError_t launch_rerank(const Shape& sh, const void* q, const void* k, const Prior& pr,
                         const int32_t* keep, const int32_t* keep_count, int keep_w, int n_lo,
                         int n_rows, int topk, int32_t* idx, float* score, void* ws,
                         size_t ws_bytes, hipStream_t st)
{
    return launch_topk(sh, q, nullptr, k, pr, keep, keep_count, keep_w, n_lo, n_rows, topk, idx,
                       score, true, ws, ws_bytes, st);
}

}  // namespace fs
