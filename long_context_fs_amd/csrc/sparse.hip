// sparse.hip -- long-range token readout with RMSNorm (FreeSolo summary,
// section 3.3, eq. 9).
//
// u_i = softmax over the tokens of the selected cells of q_i . k_j / sqrt(d)
// (unrotated, NoPE), times v_j; o_lr_i = u_i / sqrt(mean(u_i^2) + eps).
//
// bf16 storage: a workgroup owns 128 consecutive queries of one head.  It first
// builds the union of the cells they selected (an LDS bitmap over the cells,
// ranks by prefix popcount), and each query's selected cells as ascending
// union slots.  It then streams the union two cells (64 keys) at a time through
// LDS, exactly like the window kernel's key tiles, and each wave runs the
// flash tile for its 32 queries with the mask "query selected this cell"
// (a per-query bitmap over the union slots).  q and k are the exact bf16
// inputs (no rotation), so S^T = K Q^T is exact-product bf16 MFMA.  Epilogue:
// divide by the softmax sum, RMSNorm over d with a 4-lane reduction, store.
// f32 storage: the same workgroups, union and masks with fp32 K/V tiles on the
// fp32 matrix product (sparse_attn_f32_kernel).  Short query ranges split each
// tile's union over workgroups whose partial states a merge kernel combines.
// More than 32768 cells, or union bookkeeping beyond 160 KiB of LDS: one
// wavefront per query (row-wise).
#include <mutex>

#include "fs_device.hpp"
#include "fs_launch.hpp"
#include "mfma_tile.hpp"

// Scratch of the allocation-free readout (fs_sparse_attn_noalloc): the partial
// softmax states of a split readout, in device memory each GPU holds for the
// life of the process.  Host code never uses this name as an address; it uses
// the per-device pointer hipGetSymbolAddress returns (sparse_noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[fs::kSparseNoAllocBytes];

namespace fs {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

void* sparse_noalloc_scratch(hipError_t* err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    *err = hipSuccess;
    return g_scratch_ptr[dev];
}

// One wavefront per query row; lanes take two selected cells (64 tokens) at a time.
template <class E, int D>
__global__ __launch_bounds__(256) void sparse_attn_rowwise_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const typename E::storage* __restrict__ k, const typename E::storage* __restrict__ v,
    int64_t kvs0, int64_t kvs1, int64_t kvs2, int H, int nq, const int32_t* __restrict__ idx,
    int topk, float scale_log2, float rms_eps, typename E::storage* o,
    int64_t os0, int64_t os1, int64_t os2, const typename E::storage* o_sr,
    const float* __restrict__ alpha)
{
    constexpr int EPL = E::kPer16B;
    constexpr int R = D / kWave;
    __shared__ float s_q[4][D];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + wv;
    const long bh = blockIdx.y;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const bool active = row < nq;
    if (active) {
        const typename E::storage* qrow = q + b * qs0 + h * qs1 + row * qs2;
        for (int e = lane; e < D; e += kWave) s_q[wv][e] = load1<E>(qrow + e);
    }
    __syncthreads();
    if (!active) return;

    const int32_t* sel = idx + (bh * nq + row) * (long)topk;
    int n_sel = 0;
    for (int a0 = 0; a0 < topk; a0 += kWave) {
        const bool ok = a0 + lane < topk && sel[a0 + lane] >= 0;
        n_sel += __popcll(__ballot(ok));
    }
    const typename E::storage* kh = k + b * kvs0 + h * kvs1;
    const typename E::storage* vh = v + b * kvs0 + h * kvs1;
    const float* qv = s_q[wv];

    float m = -INFINITY, l = 0.f, acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    for (int a0 = 0; a0 < n_sel; a0 += 2) {
        const int a = a0 + (lane >> 5);
        const bool valid = a < n_sel;
        long j = 0;
        float s = -INFINITY;
        if (valid) {
            j = (long)sel[a] * 32 + (lane & 31);
            const typename E::storage* kr = kh + j * kvs2;
            float dot = 0.f;
            for (int e0 = 0; e0 < D; e0 += EPL) {
                float x[EPL];
                load16<E>(kr + e0, x);
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e0 + e], x[e], dot);
            }
            s = dot * scale_log2;
        }
        const float m_new = fmaxf(m, wave_max(s));
        const float corr = exp2f(m - m_new);
        const float p = valid ? exp2f(s - m_new) : 0.f;
        l = l * corr + wave_sum(p);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] *= corr;
        const int cnt = (n_sel - a0) >= 2 ? kWave : 32;
        for (int jj = 0; jj < cnt; ++jj) {
            const float pj = __shfl(p, jj, kWave);
            const long jt = (long)sel[a0 + (jj >> 5)] * 32 + (jj & 31);
            const typename E::storage* vr = vh + jt * kvs2;
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = fmaf(pj, load1<E>(vr + lane + r * kWave), acc[r]);
        }
        m = m_new;
    }
    float u[R], ss = 0.f;
    const float inv_l = n_sel > 0 ? 1.f / l : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        u[r] = acc[r] * inv_l;
        ss = fmaf(u[r], u[r], ss);
    }
    ss = wave_sum(ss);
    const float inv_rms = 1.f / sqrtf(ss / (float)D + rms_eps);
    typename E::storage* orow = o + b * os0 + h * os1 + row * os2;
    if (o_sr) {                        // eq. 2 in the epilogue: o = o_sr + alpha_h o_lr
        const typename E::storage* srow = o_sr + b * os0 + h * os1 + row * os2;
        const float a = alpha[h];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float x = load1<E>(srow + lane + r * kWave);
            store1<E>(orow + lane + r * kWave, fmaf(a, u[r] * inv_rms, x));
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) store1<E>(orow + lane + r * kWave, u[r] * inv_rms);
}


namespace {

constexpr int kSpQ = 128;              // queries per workgroup
constexpr int kSpMaxCells = 32768;     // bitmap capacity (cells), so N <= 1M tokens

// LDS of the union-masked readout.  Besides the K / V^T tile: the union bitmap
// over cells, its per-word ranks, the union list (slot -> cell) and, per query,
// a bitmap over union slots of the cells that query selected (odd pitch, so the
// 16 queries of a lane row read distinct banks).
struct SpLayout {
    int nwords, u_cap, qpitch;
    size_t off_vt, off_bitmap, off_rank, off_ulist, off_qbits, bytes;
};

// F32: fp32 K and V tiles, row-major with rows padded by kSpF32Pad floats.
constexpr int kSpF32Pad = 4;

template <int D, bool F32 = false>
__host__ __device__ inline SpLayout sp_layout(int C, int topk)
{
    SpLayout L;
    L.nwords = (C + 31) / 32;
    L.u_cap = C < kSpQ * topk ? C : kSpQ * topk;
    L.qpitch = ((L.u_cap + 31) / 32) | 1;
    auto up16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
    const size_t tile = F32 ? (size_t)mf::kTileK * (D + kSpF32Pad) * 4 : (size_t)mf::kTileK * D * 2;
    size_t off = tile;                                   // K tile (swizzled bf16, or fp32 rows)
    L.off_vt = off;
    off = up16(off + tile);                              // V^T tile (bf16), or V rows (fp32)
    L.off_bitmap = off;
    off = up16(off + (size_t)L.nwords * 4);
    L.off_rank = off;
    off = up16(off + (size_t)L.nwords * 2);
    L.off_ulist = off;
    off = up16(off + (size_t)L.u_cap * 2);
    L.off_qbits = off;
    off = up16(off + (size_t)kSpQ * L.qpitch * 4);
    L.bytes = off;
    return L;
}

// Block-wide exclusive scan of one int per thread (256 threads); *total = sum.
__device__ __forceinline__ int block_excl_scan(int x, int* red, int* total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int inc = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
    }
    if (lane == kWave - 1) red[wv] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < wv) before += red[i];
        all += red[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

// The union of the cells the tile's queries selected: bitmap over the cells,
// per-word ranks, the slot -> cell list, and per query a bitmap over the union
// slots it selected.  Returns the union's size (block-uniform); ends with a
// barrier.
__device__ __forceinline__ int sp_union(const SpLayout& L, uint32_t* bitmap, uint16_t* rank,
                                        uint16_t* ulist, uint32_t* qbits,
                                        const int32_t* __restrict__ idx_blk, int n_rows, int topk,
                                        int C, int* red)
{
    const int tid = threadIdx.x;
    for (int wd = tid; wd < L.nwords; wd += 256) bitmap[wd] = 0u;
    for (int e = tid; e < kSpQ * L.qpitch; e += 256) qbits[e] = 0u;
    __syncthreads();
    for (int e = tid; e < n_rows * topk; e += 256) {
        const int c = idx_blk[e];
        if (c >= 0 && c < C) atomicOr(&bitmap[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    int cnt[4], mine = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int wd = 4 * tid + j;
        cnt[j] = wd < L.nwords ? __popc(bitmap[wd]) : 0;
        mine += cnt[j];
    }
    int n_union;
    int run = block_excl_scan(mine, red, &n_union);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int wd = 4 * tid + j;
        if (wd < L.nwords) rank[wd] = (uint16_t)run;
        run += cnt[j];
    }
    __syncthreads();
    for (int wd = tid; wd < L.nwords; wd += 256) {
        uint32_t bits = bitmap[wd];
        int r = rank[wd];
        while (bits) {
            const int bpos = __ffs(bits) - 1;
            ulist[r++] = (uint16_t)(32 * wd + bpos);
            bits &= bits - 1;
        }
    }
    for (int e = tid; e < n_rows * topk; e += 256) {
        const int c = idx_blk[e];
        if (c >= 0 && c < C) {
            const int sl = rank[c >> 5] + __popc(bitmap[c >> 5] & ((1u << (c & 31)) - 1u));
            atomicOr(&qbits[(e / topk) * L.qpitch + (sl >> 5)], 1u << (sl & 31));
        }
    }
    __syncthreads();
    return n_union;
}

// Register stage of one 64-key tile (two cells): KC 16-byte chunks of K rows
// per thread, and for threads t < 2D four keys x 8 dims of V.  Every chunk a
// wave loads lies in one cell, so a load is a wave-uniform cell base plus a
// per-lane byte offset fixed for the whole kernel.
template <int D>
struct SpStage {
    static constexpr int KC = (mf::kTileK * D / 8) / 256;
    uint4 k[KC];
    uint4 v[4];
};

// Per-lane byte offsets of the stage loads within a cell: thread t's K chunk of
// stage slot `it` sits at kbase + row(it) * row_bytes, where row(it) is uniform;
// its V rows at vbase + r * row_bytes, in cell vgrp = t / D (uniform per wave).
template <int D>
struct SpOffsets {
    uint32_t kbase, vbase;
    int vgrp;
    bool has_v;
};

template <int D>
__device__ __forceinline__ SpOffsets<D> sp_offsets(int64_t kvs2)
{
    SpOffsets<D> o;
    const int tid = threadIdx.x;
    o.kbase = (uint32_t)(((tid / (D / 8)) * kvs2 + (tid % (D / 8)) * 8) * 2);
    const int within = tid % D, hh = within & 1, g = (within >> 1) & 3, dc = within >> 3;
    o.vbase = (uint32_t)(((16 * hh + 4 * g) * kvs2 + dc * 8) * 2);
    o.vgrp = __builtin_amdgcn_readfirstlane(tid / D);          // wave-uniform
    o.has_v = __builtin_amdgcn_readfirstlane(tid < 2 * D) != 0;
    return o;
}

// Stage slot `it` holds key rows (tid / (D/8)) + it * 2048 / D of the 64-key tile:
// cell (it * 2048 / D) / 32, row (it * 2048 / D) % 32 of that cell plus the lane's own.
template <int D>
__host__ __device__ constexpr int sp_kchunk_cell(int it) { return it * (2048 / D) / 32; }
template <int D>
__host__ __device__ constexpr int sp_kchunk_row(int it) { return it * (2048 / D) % 32; }

template <int D>
__device__ __forceinline__ void sp_load(SpStage<D>& st, const SpOffsets<D>& o, const char* kh,
                                        const char* vh, int64_t kvs2,
                                        const uint16_t* ulist, int n_union, int u)
{
    // the tile's two cells; past the end of an odd union the second repeats the
    // first (its keys are then masked for every query)
    const int64_t row_bytes = kvs2 * 2, cell_bytes = 32 * row_bytes;
    const int c0 = __builtin_amdgcn_readfirstlane(ulist[2 * u]);
    const int c1 = __builtin_amdgcn_readfirstlane(2 * u + 1 < n_union ? ulist[2 * u + 1] : c0);
#pragma unroll
    for (int it = 0; it < SpStage<D>::KC; ++it) {
        const char* cb = kh + (sp_kchunk_cell<D>(it) ? c1 : c0) * cell_bytes +
                         sp_kchunk_row<D>(it) * row_bytes;
        st.k[it] = *reinterpret_cast<const uint4*>(cb + o.kbase);
    }
    if (o.has_v) {
        const char* vb = vh + (o.vgrp ? c1 : c0) * cell_bytes;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st.v[r] = *reinterpret_cast<const uint4*>(vb + r * row_bytes + o.vbase);
    }
}

template <int D>
__device__ __forceinline__ void sp_store(const SpStage<D>& st, uint16_t* ks, uint16_t* vt)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < SpStage<D>::KC; ++it) {
        const int c = tid + 256 * it;
        const int kr = c / (D / 8), part = c % (D / 8);
        mf::lds_store16(ks + mf::ksw_off<D>(kr, part), st.k[it]);
    }
    if (tid < 2 * D) {
        const int grp = tid / D, within = tid % D;
        const int hh = within & 1, g = (within >> 1) & 3, dc = within >> 3;
        mf::store_vt_4x8_sw(st.v, vt, dc, 32 * grp + 8 * g + 4 * hh);
    }
}

// One 64-key tile (two cells of 32 keys) for a wave's 32 queries.  sel[qg][c]
// says whether query 16 qg + n selected the tile's cell c.  A cell's scores are
// masked through the exponent bias (-inf for a cell the query did not select),
// so no score is touched twice; the softmax denominator is accumulated on the
// matrix core as P^T times a row of ones, from the same bf16 weights as O.
template <int D>
__device__ __forceinline__ void sp_tile(const uint16_t* ks, const uint16_t* vt,
                                        const mf::bf16x8 (&qf)[2][D / 32],
                                        mf::f32x4 (&acc)[D / 16][2], mf::f32x4 (&accl)[2],
                                        float (&m_ref)[2], float scale_log2,
                                        const bool (&sel)[2][2])
{
    using namespace mf;
    constexpr int KS = D / 32, DB = D / 16;
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 a = as_bf16x8(lds_load16(ks + ksw_off<D>(16 * kb + n, 4 * t + g)));
            s[kb][0] = mfma(a, qf[0][t], s[kb][0]);
            s[kb][1] = mfma(a, qf[1][t], s[kb][1]);
        }
    }
    bf16x8 pf[2][2];
    float corr[2];
    bool any_rescale = false;
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        float cm[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float x = -INFINITY;
#pragma unroll
            for (int kb = 2 * c; kb < 2 * c + 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)   // IEEE maximum: no NaN quieting of MFMA results
                    x = __builtin_elementwise_maximum(x, s[kb][qg][r]);
            cm[c] = sel[qg][c] ? x : -INFINITY;
        }
        // scale_log2 > 0 commutes with max
        const float tmax = xrow_max(__builtin_elementwise_maximum(cm[0], cm[1])) * scale_log2;
        const bool raise = tmax > m_ref[qg] + kLazy;
        const float m_new = raise ? tmax : m_ref[qg];
        corr[qg] = raise ? __builtin_amdgcn_exp2f(m_ref[qg] - m_new) : 1.f;   // 0 at the start
        any_rescale |= raise;
        m_ref[qg] = m_new;
        // a selected cell implies a finite m_new; an unselected one gets p = 0
        float bias[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) bias[c] = sel[qg][c] ? -m_new : -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s[kb][qg][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qg][r], scale_log2, bias[kb >> 1]));
        pf[0][qg] = pack_p(s[0][qg], s[1][qg]);
        pf[1][qg] = pack_p(s[2][qg], s[3][qg]);
    }
    if (__builtin_expect(__ballot(any_rescale) != 0, 0)) {
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db][qg] *= corr[qg];
            accl[qg] *= corr[qg];
        }
    }
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
            const bf16x8 a = as_bf16x8(lds_load16(vt + vtsw_off(16 * db + n, 4 * a2 + g)));
            acc[db][0] = mfma(a, pf[a2][0], acc[db][0]);
            acc[db][1] = mfma(a, pf[a2][1], acc[db][1]);
        }
    }
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
        accl[0] = mfma(ones, pf[a2][0], accl[0]);
        accl[1] = mfma(ones, pf[a2][1], accl[1]);
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void sparse_attn_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t kvs0, int64_t kvs1,
    int64_t kvs2, int H, int BH, int nq, int C, const int32_t* __restrict__ idx, int topk,
    float scale_log2, float rms_eps, uint16_t* o, int64_t os0, int64_t os1,
    int64_t os2, int n_split, float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
    const uint16_t* o_sr, const float* __restrict__ alpha)
{
    using namespace mf;
    constexpr int KS = D / 32, DB = D / 16;
    extern __shared__ uint4 smem_raw[];
    const SpLayout L = sp_layout<D>(C, topk);
    char* base = reinterpret_cast<char*>(smem_raw);
    uint16_t* ks = reinterpret_cast<uint16_t*>(base);
    uint16_t* vt = reinterpret_cast<uint16_t*>(base + L.off_vt);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.off_bitmap);
    uint16_t* rank = reinterpret_cast<uint16_t*>(base + L.off_rank);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(base + L.off_ulist);
    uint32_t* qbits = reinterpret_cast<uint32_t*>(base + L.off_qbits);
    __shared__ int red[4];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    // workgroup -> (head, split, query tile); the head is the fastest index (XCD locality)
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int split = (int)(tb.tile % n_split);
    const int h = (int)(bh % H), b = (int)(bh / H);
    const long t0 = (tb.tile / n_split) * kSpQ;
    const int n_rows = nq - t0 < kSpQ ? (int)(nq - t0) : kSpQ;
    const int32_t* idx_blk = idx + (bh * nq + t0) * (long)topk;

    // ---- union of the selected cells, and each query's selection over it ----
    const int n_union = sp_union(L, bitmap, rank, ulist, qbits, idx_blk, n_rows, topk, C, red);

    // ---- queries of this wave as B operands -------------------------------
    const char* kh = reinterpret_cast<const char*>(k + b * kvs0 + h * kvs1);
    const char* vh = reinterpret_cast<const char*>(v + b * kvs0 + h * kvs1);
    bf16x8 qf[2][KS];
    const int qbit_row = (32 * wv + n) * L.qpitch;   // query group 1 is 16 rows further
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int r = 32 * wv + 16 * qg + n;
        const bool ok = r < n_rows;
        const uint16_t* qrow = q + b * qs0 + h * qs1 + (t0 + (ok ? r : 0)) * qs2;
#pragma unroll
        for (int t = 0; t < KS; ++t)
            qf[qg][t] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * g)
                                     : make_uint4(0, 0, 0, 0));
    }

    f32x4 acc[DB][2], accl[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    accl[0] = accl[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};

    const SpOffsets<D> offs = sp_offsets<D>(kvs2);
    // this workgroup's share of the union's 64-key tiles
    const int n_all = (n_union + 1) / 2;
    const int u_begin = (int)((long)n_all * split / n_split);
    const int u_end = (int)((long)n_all * (split + 1) / n_split);
    SpStage<D> stage;
    if (u_begin < u_end) {
        sp_load<D>(stage, offs, kh, vh, kvs2, ulist, n_union, u_begin);
        sp_store<D>(stage, ks, vt);
    }
    __syncthreads();
    uint32_t qw[2] = {0u, 0u};
    for (int u = u_begin; u < u_end; ++u) {
        if (u + 1 < u_end) sp_load<D>(stage, offs, kh, vh, kvs2, ulist, n_union, u + 1);
        if ((u & 15) == 0 || u == u_begin) {
            qw[0] = qbits[qbit_row + (u >> 4)];                  // rows past n_rows are zero
            qw[1] = qbits[qbit_row + 16 * L.qpitch + (u >> 4)];
        }
        const int sh = (2 * u) & 31;
        const bool sel[2][2] = {{((qw[0] >> sh) & 1u) != 0, ((qw[0] >> (sh + 1)) & 1u) != 0},
                                {((qw[1] >> sh) & 1u) != 0, ((qw[1] >> (sh + 1)) & 1u) != 0}};
        if (__ballot(sel[0][0] || sel[0][1] || sel[1][0] || sel[1][1]) != 0)
            sp_tile<D>(ks, vt, qf, acc, accl, m_run, scale_log2, sel);
        __syncthreads();
        if (u + 1 < u_end) {
            sp_store<D>(stage, ks, vt);
            __syncthreads();
        }
    }

    if (n_split > 1) {
        // ---- partial softmax state of this split: (m, l) and the unnormalised O
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const int r = 32 * wv + 16 * qg + n;
            if (r >= n_rows) continue;
            const long slot = (bh * nq + t0 + r) * n_split + split;
            if (g == 0) ws_ml[slot] = make_float2(m_run[qg], accl[qg][0]);
            float* a = ws_acc + slot * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *reinterpret_cast<f32x4*>(a + 16 * db + 4 * g) = acc[db][qg];
        }
        return;
    }

    // ---- epilogue: normalise, RMSNorm over d, store ------------------------
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int r = 32 * wv + 16 * qg + n;
        const float l = accl[qg][0];    // every row of the ones product is the full sum
        const float inv_l = l > 0.f ? 1.f / l : 0.f;
        float ss = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            acc[db][qg] *= inv_l;
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = fmaf(acc[db][qg][e], acc[db][qg][e], ss);
        }
        ss = xrow_sum(ss);
        const float inv_rms = 1.f / sqrtf(ss / (float)D + rms_eps);
        if (r >= n_rows) continue;
        uint16_t* orow = o + b * os0 + h * os1 + (t0 + r) * os2;
        if (o_sr) {                    // eq. 2 in the epilogue: o = o_sr + alpha_h o_lr
            const uint16_t* srow = o_sr + b * os0 + h * os1 + (t0 + r) * os2;
            const float a = alpha[h];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint2 x2 = *reinterpret_cast<const uint2*>(srow + 16 * db + 4 * g);
                uint2 w2;
                w2.x = cvt_pk_bf16(fmaf(a, acc[db][qg][0] * inv_rms, __uint_as_float(x2.x << 16)),
                                   fmaf(a, acc[db][qg][1] * inv_rms,
                                        __uint_as_float(x2.x & 0xFFFF0000u)));
                w2.y = cvt_pk_bf16(fmaf(a, acc[db][qg][2] * inv_rms, __uint_as_float(x2.y << 16)),
                                   fmaf(a, acc[db][qg][3] * inv_rms,
                                        __uint_as_float(x2.y & 0xFFFF0000u)));
                *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g) = w2;
            }
            continue;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            uint2 w2;
            w2.x = cvt_pk_bf16(acc[db][qg][0] * inv_rms, acc[db][qg][1] * inv_rms);
            w2.y = cvt_pk_bf16(acc[db][qg][2] * inv_rms, acc[db][qg][3] * inv_rms);
            *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g) = w2;
        }
    }
}

// fp32 storage on the matrix core: the bf16 kernel's workgroups, union, masks
// and splits, with fp32 K / V tiles (rows padded against bank conflicts) and
// the fp32 product v_mfma_f32_16x16x4f32.  As in the fp32 window, the QK^T
// contraction gives lane group g dimensions g*D/4 .. g*D/4 + D/4 - 1 (contiguous
// reads), and PV step j of a 16-key block contracts keys 4g + j, register j of
// the lane's S^T fragment; V needs no transposition.
namespace {

template <int D>
struct SpStageF32 {
    static constexpr int KC = (mf::kTileK * D / 4) / 256;   // 16-byte chunks per thread
    mf::f32x4 k[KC];   // native vectors: a float4 struct copy would stay in scratch
    mf::f32x4 v[KC];
};

template <int D>
__device__ __forceinline__ void spf_load(SpStageF32<D>& st, const float* kh, const float* vh,
                                         int64_t kvs2, const uint16_t* ulist, int n_union, int u)
{
    // the tile's two cells; past the end of an odd union the second repeats the
    // first (its keys are then masked for every query)
    const int c0 = __builtin_amdgcn_readfirstlane(ulist[2 * u]);
    const int c1 = __builtin_amdgcn_readfirstlane(2 * u + 1 < n_union ? ulist[2 * u + 1] : c0);
#pragma unroll
    for (int it = 0; it < SpStageF32<D>::KC; ++it) {
        const int f = threadIdx.x + 256 * it;
        const int kr = f / (D / 4), part = f % (D / 4);
        const long row = (long)(kr < 32 ? c0 : c1) * 32 + (kr & 31);
        st.k[it] = *reinterpret_cast<const mf::f32x4*>(kh + row * kvs2 + part * 4);
        st.v[it] = *reinterpret_cast<const mf::f32x4*>(vh + row * kvs2 + part * 4);
    }
}

template <int D>
__device__ __forceinline__ void spf_store(const SpStageF32<D>& st, float* ks, float* vs)
{
    constexpr int P = D + kSpF32Pad;
#pragma unroll
    for (int it = 0; it < SpStageF32<D>::KC; ++it) {
        const int f = threadIdx.x + 256 * it;
        const int kr = f / (D / 4), part = f % (D / 4);
        *reinterpret_cast<mf::f32x4*>(ks + kr * P + part * 4) = st.k[it];
        *reinterpret_cast<mf::f32x4*>(vs + kr * P + part * 4) = st.v[it];
    }
}

}  // namespace

// d128's registers (2 x 32 query floats, 2 x 32 accumulators, a 32 KiB tile
// stage) fit one wave per SIMD.
template <int D>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void sparse_attn_f32_kernel(
    const float* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ k, const float* __restrict__ v, int64_t kvs0, int64_t kvs1,
    int64_t kvs2, int H, int BH, int nq, int C, const int32_t* __restrict__ idx, int topk,
    float scale_log2, float rms_eps, float* o, int64_t os0, int64_t os1, int64_t os2,
    int n_split, float* __restrict__ ws_acc, float2* __restrict__ ws_ml, const float* o_sr,
    const float* __restrict__ alpha)
{
    using namespace mf;
    constexpr int T = D / 4, DB = D / 16, P = D + kSpF32Pad;
    extern __shared__ uint4 smem_raw[];
    const SpLayout L = sp_layout<D, true>(C, topk);
    char* base = reinterpret_cast<char*>(smem_raw);
    float* ks = reinterpret_cast<float*>(base);
    float* vs = reinterpret_cast<float*>(base + L.off_vt);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + L.off_bitmap);
    uint16_t* rank = reinterpret_cast<uint16_t*>(base + L.off_rank);
    uint16_t* ulist = reinterpret_cast<uint16_t*>(base + L.off_ulist);
    uint32_t* qbits = reinterpret_cast<uint32_t*>(base + L.off_qbits);
    __shared__ int red[4];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int split = (int)(tb.tile % n_split);
    const int h = (int)(bh % H), b = (int)(bh / H);
    const long t0 = (tb.tile / n_split) * kSpQ;
    const int n_rows = nq - t0 < kSpQ ? (int)(nq - t0) : kSpQ;
    const int32_t* idx_blk = idx + (bh * nq + t0) * (long)topk;
    const int n_union = sp_union(L, bitmap, rank, ulist, qbits, idx_blk, n_rows, topk, C, red);

    const float* kh = k + b * kvs0 + h * kvs1;
    const float* vh = v + b * kvs0 + h * kvs1;
    float qf[2][T];                                  // dims g*T .. g*T+T-1 of query 16 qg + n
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int r = 32 * wv + 16 * qg + n;
        const bool ok = r < n_rows;
        const float* qrow = q + b * qs0 + h * qs1 + (t0 + (ok ? r : 0)) * qs2 + g * T;
#pragma unroll
        for (int c = 0; c < T / 4; ++c) {
            const float4 x = ok ? *reinterpret_cast<const float4*>(qrow + 4 * c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            qf[qg][4 * c + 0] = x.x;
            qf[qg][4 * c + 1] = x.y;
            qf[qg][4 * c + 2] = x.z;
            qf[qg][4 * c + 3] = x.w;
        }
    }

    f32x4 acc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float l_part[2] = {0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    const int qbit_row = (32 * wv + n) * L.qpitch;

    const int n_all = (n_union + 1) / 2;
    const int u_begin = (int)((long)n_all * split / n_split);
    const int u_end = (int)((long)n_all * (split + 1) / n_split);
    SpStageF32<D> stage;
    if (u_begin < u_end) {
        spf_load<D>(stage, kh, vh, kvs2, ulist, n_union, u_begin);
        spf_store<D>(stage, ks, vs);
    }
    __syncthreads();
    uint32_t qw[2] = {0u, 0u};
    for (int u = u_begin; u < u_end; ++u) {
        if (u + 1 < u_end) spf_load<D>(stage, kh, vh, kvs2, ulist, n_union, u + 1);
        if ((u & 15) == 0 || u == u_begin) {
            qw[0] = qbits[qbit_row + (u >> 4)];
            qw[1] = qbits[qbit_row + 16 * L.qpitch + (u >> 4)];
        }
        const int sh = (2 * u) & 31;
        const bool sel[2][2] = {{((qw[0] >> sh) & 1u) != 0, ((qw[0] >> (sh + 1)) & 1u) != 0},
                                {((qw[1] >> sh) & 1u) != 0, ((qw[1] >> (sh + 1)) & 1u) != 0}};
        if (__ballot(sel[0][0] || sel[0][1] || sel[1][0] || sel[1][1]) != 0) {
            f32x4 s[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                const float* krow = ks + (16 * kb + n) * P + g * T;
#pragma unroll
                for (int c = 0; c < T / 4; ++c) {
                    const float4 a = *reinterpret_cast<const float4*>(krow + 4 * c);
                    s[kb][0] = mfma_f32(a.x, qf[0][4 * c + 0], s[kb][0]);
                    s[kb][1] = mfma_f32(a.x, qf[1][4 * c + 0], s[kb][1]);
                    s[kb][0] = mfma_f32(a.y, qf[0][4 * c + 1], s[kb][0]);
                    s[kb][1] = mfma_f32(a.y, qf[1][4 * c + 1], s[kb][1]);
                    s[kb][0] = mfma_f32(a.z, qf[0][4 * c + 2], s[kb][0]);
                    s[kb][1] = mfma_f32(a.z, qf[1][4 * c + 2], s[kb][1]);
                    s[kb][0] = mfma_f32(a.w, qf[0][4 * c + 3], s[kb][0]);
                    s[kb][1] = mfma_f32(a.w, qf[1][4 * c + 3], s[kb][1]);
                }
            }
            float corr[2];
            bool any_rescale = false;
#pragma unroll
            for (int qg = 0; qg < 2; ++qg) {
                float cm[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float x = -INFINITY;
#pragma unroll
                    for (int kb = 2 * c; kb < 2 * c + 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            x = __builtin_elementwise_maximum(x, s[kb][qg][r]);
                    cm[c] = sel[qg][c] ? x : -INFINITY;
                }
                const float tmax =
                    xrow_max(__builtin_elementwise_maximum(cm[0], cm[1])) * scale_log2;
                const bool raise = tmax > m_run[qg] + kLazy;
                const float m_new = raise ? tmax : m_run[qg];
                corr[qg] = raise ? __builtin_amdgcn_exp2f(m_run[qg] - m_new) : 1.f;
                any_rescale |= raise;
                m_run[qg] = m_new;
                float bias[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) bias[c] = sel[qg][c] ? -m_new : -INFINITY;
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        s[kb][qg][r] =
                            __builtin_amdgcn_exp2f(fmaf(s[kb][qg][r], scale_log2, bias[kb >> 1]));
                        ls += s[kb][qg][r];
                    }
                l_part[qg] = fmaf(l_part[qg], corr[qg], ls);
            }
            if (__builtin_expect(__ballot(any_rescale) != 0, 0)) {
#pragma unroll
                for (int qg = 0; qg < 2; ++qg)
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[db][qg] *= corr[qg];
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float a = vs[(16 * kb + 4 * g + j) * P + 16 * db + n];
                        acc[db][0] = mfma_f32(a, s[kb][0][j], acc[db][0]);
                        acc[db][1] = mfma_f32(a, s[kb][1][j], acc[db][1]);
                    }
                }
            }
        }
        __syncthreads();
        if (u + 1 < u_end) {
            spf_store<D>(stage, ks, vs);
            __syncthreads();
        }
    }

    float l[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) l[qg] = xrow_sum(l_part[qg]);
    if (n_split > 1) {
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const int r = 32 * wv + 16 * qg + n;
            if (r >= n_rows) continue;
            const long slot = (bh * nq + t0 + r) * n_split + split;
            if (g == 0) ws_ml[slot] = make_float2(m_run[qg], l[qg]);
            float* a = ws_acc + slot * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *reinterpret_cast<f32x4*>(a + 16 * db + 4 * g) = acc[db][qg];
        }
        return;
    }
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const int r = 32 * wv + 16 * qg + n;
        const float inv_l = l[qg] > 0.f ? 1.f / l[qg] : 0.f;
        float ss = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            acc[db][qg] *= inv_l;
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = fmaf(acc[db][qg][e], acc[db][qg][e], ss);
        }
        ss = xrow_sum(ss);
        const float inv_rms = 1.f / sqrtf(ss / (float)D + rms_eps);
        if (r >= n_rows) continue;
        float* orow = o + b * os0 + h * os1 + (t0 + r) * os2;
        if (o_sr) {                    // eq. 2 in the epilogue: o = o_sr + alpha_h o_lr
            const float* srow = o_sr + b * os0 + h * os1 + (t0 + r) * os2;
            const float a = alpha[h];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const float4 x = *reinterpret_cast<const float4*>(srow + 16 * db + 4 * g);
                *reinterpret_cast<float4*>(orow + 16 * db + 4 * g) =
                    make_float4(fmaf(a, acc[db][qg][0] * inv_rms, x.x),
                                fmaf(a, acc[db][qg][1] * inv_rms, x.y),
                                fmaf(a, acc[db][qg][2] * inv_rms, x.z),
                                fmaf(a, acc[db][qg][3] * inv_rms, x.w));
            }
            continue;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<float4*>(orow + 16 * db + 4 * g) =
                make_float4(acc[db][qg][0] * inv_rms, acc[db][qg][1] * inv_rms,
                            acc[db][qg][2] * inv_rms, acc[db][qg][3] * inv_rms);
    }
}

// Merge of a split attention (the readout, or the window branch): per query, the
// partial states (m_s, l_s, O_s) (reference maxima in the log2 domain) combine as
// O = sum_s 2^(m_s - M) O_s over l = sum_s 2^(m_s - M) l_s with M = max_s m_s;
// then RMSNorm when RMS (the readout, eq. 9).  One wavefront per query, D / 64
// dims per lane.
template <class E, int D, bool RMS>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ ws_acc,
                                                           const float2* __restrict__ ws_ml,
                                                           int H, int nq, long n_rows_all,
                                                           int n_split, float rms_eps,
                                                           typename E::storage* o, int64_t os0,
                                                           int64_t os1, int64_t os2,
                                                           const typename E::storage* o_sr,
                                                           const float* __restrict__ alpha)
{
    constexpr int R = D / kWave;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);    // = bh * nq + t
    if (row >= n_rows_all) return;
    const int lane = threadIdx.x & 63;
    // lane sp holds split sp's (m, l) (n_split <= 32): one max and one sum over the wave
    const float2 e = lane < n_split ? ws_ml[row * n_split + lane] : make_float2(-INFINITY, 0.f);
    const float M = wave_max(e.x);
    const float w = (M != -INFINITY && lane < n_split) ? __builtin_amdgcn_exp2f(e.x - M) : 0.f;
    const float l = wave_sum(w * e.y);                    // an empty split has weight 0
    float acc[R] = {};
    if (M != -INFINITY) {
        // all splits' loads issued at once: a split past n_split re-reads the last
        // one and has weight 0, so the loop has no branch
        const float* a = ws_acc + row * n_split * (long)D + lane;
        float x[32][R];
#pragma unroll
        for (int sp = 0; sp < 32; ++sp)
#pragma unroll
            for (int r = 0; r < R; ++r)
                x[sp][r] = a[(sp < n_split ? sp : n_split - 1) * D + r * kWave];
#pragma unroll
        for (int sp = 0; sp < 32; ++sp) {
            const float ws = __shfl(w, sp, kWave);          // 0 for sp >= n_split
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = fmaf(ws, x[sp][r], acc[r]);
        }
    }
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] *= inv_l;
        ss = fmaf(acc[r], acc[r], ss);
    }
    float inv_rms = 1.f;
    if constexpr (RMS) inv_rms = 1.f / sqrtf(wave_sum(ss) / (float)D + rms_eps);
    const long bh = row / nq, t = row - bh * nq;
    const int h = (int)(bh % H), b = (int)(bh / H);
    typename E::storage* orow = o + b * os0 + h * os1 + t * os2;
    if (o_sr) {                        // eq. 2 in the epilogue: o = o_sr + alpha_h o_lr
        const typename E::storage* srow = o_sr + b * os0 + h * os1 + t * os2;
        const float a = alpha[h];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float x = load1<E>(srow + lane + r * kWave);
            store1<E>(orow + lane + r * kWave, fmaf(a, acc[r] * inv_rms, x));
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) store1<E>(orow + lane + r * kWave, acc[r] * inv_rms);
}

hipError_t launch_split_merge(const Shape& sh, int S, const float* ws_acc, const float2* ws_ml,
                              bool rms, float rms_eps, void* o, hipStream_t st, const void* o_sr,
                              const float* alpha)
{
    const long rows_all = (long)sh.B * sh.H * sh.nq;
    dim3 mgrid((unsigned)((rows_all + 3) / 4));
#define FS_MERGE(E, D, RMS)                                                                       \
    hipLaunchKernelGGL((split_merge_kernel<E, D, RMS>), mgrid, dim3(256), 0, st, ws_acc, ws_ml,   \
                       sh.H, sh.nq, rows_all, S, rms_eps, (typename E::storage*)o, sh.os[0],     \
                       sh.os[1], sh.os[2], (const typename E::storage*)o_sr, alpha)
    if (sh.bf16) {
        if (sh.d == 64) {
            if (rms) FS_MERGE(Bf16, 64, true); else FS_MERGE(Bf16, 64, false);
        } else {
            if (rms) FS_MERGE(Bf16, 128, true); else FS_MERGE(Bf16, 128, false);
        }
    } else {
        if (sh.d == 64) {
            if (rms) FS_MERGE(F32, 64, true); else FS_MERGE(F32, 64, false);
        } else {
            if (rms) FS_MERGE(F32, 128, true); else FS_MERGE(F32, 128, false);
        }
    }
#undef FS_MERGE
    return hipGetLastError();
}

// Split count: about one workgroup per CU in all (256), at most 32 per query tile.
// A second workgroup per CU does not pay: each split's partial state is written
// and merged, and the two share the CU's LDS and matrix cores (at 256 decode
// queries over 8 heads, 16 splits take 0.037 ms, 20-32 splits 0.053 ms).
constexpr long kSpSplitWorkgroups = 256;
static_assert(kSparseNoAllocBytes >= (size_t)kSpSplitWorkgroups * kSpQ * (128 * sizeof(float) + 8),
              "the allocation-free readout's array holds the largest split state");

int sparse_splits(const Shape& sh)
{
    if (sh.C > kSpMaxCells || sh.nq == 0) return 1;
    const long base = (sh.nq + kSpQ - 1) / kSpQ * (long)sh.B * sh.H;
    const long want = kSpSplitWorkgroups / base;
    return (int)(want < 1 ? 1 : want < 32 ? want : 32);
}

size_t sparse_ws_bytes(const Shape& sh)
{
    const int S = sparse_splits(sh);
    if (S <= 1) return 0;
    const size_t rows = (size_t)sh.B * sh.H * sh.nq * S;
    return rows * ((size_t)sh.d * sizeof(float) + sizeof(float2));
}

hipError_t launch_sparse(const Shape& sh, const void* q, const void* k, const void* v,
                         const int32_t* idx, int topk, float rms_eps, void* ws, void* o_lr,
                         hipStream_t st, const void* o_sr, const float* alpha)
{
    if (sh.nq == 0) return hipSuccess;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)sh.d));
    if (!sh.bf16) {
        const size_t lds32 = sh.d == 64 ? sp_layout<64, true>(sh.C, topk).bytes
                                        : sp_layout<128, true>(sh.C, topk).bytes;
        if (sh.C <= kSpMaxCells && lds32 <= 160 * 1024) {
            const int S = ws ? sparse_splits(sh) : 1;
            const long rows_all = (long)sh.B * sh.H * sh.nq;
            float* ws_acc = S > 1 ? static_cast<float*>(ws) : nullptr;
            float2* ws_ml =
                S > 1 ? reinterpret_cast<float2*>(ws_acc + rows_all * S * sh.d) : nullptr;
            const long n_tiles = (sh.nq + kSpQ - 1) / kSpQ;
            note_path("readout: fp32 MFMA tiles of 128 queries over their union, %d split(s)", S);
            dim3 grid((unsigned)(n_tiles * S * sh.B * sh.H)), block(256);
#define FS_SPARSE_F32(D)                                                                          \
            hipLaunchKernelGGL((sparse_attn_f32_kernel<D>), grid, block, lds32, st,               \
                               (const float*)q, sh.qs[0], sh.qs[1], sh.qs[2], (const float*)k,    \
                               (const float*)v, sh.kvs[0], sh.kvs[1], sh.kvs[2], sh.H,            \
                               sh.B * sh.H, sh.nq, sh.C, idx, topk, scale_log2, rms_eps,          \
                               (float*)o_lr, sh.os[0], sh.os[1], sh.os[2], S, ws_acc, ws_ml,      \
                               (const float*)o_sr, alpha)
            if (sh.d == 64) FS_SPARSE_F32(64); else FS_SPARSE_F32(128);
#undef FS_SPARSE_F32
            hipError_t err = hipGetLastError();
            if (err != hipSuccess || S <= 1) return err;
            return launch_split_merge(sh, S, ws_acc, ws_ml, true, rms_eps, o_lr, st, o_sr, alpha);
        }
    }
    const size_t lds = sh.d == 64 ? sp_layout<64>(sh.C, topk).bytes
                                  : sp_layout<128>(sh.C, topk).bytes;
    if (sh.bf16 && sh.C <= kSpMaxCells && lds <= 160 * 1024) {
        const int S = ws ? sparse_splits(sh) : 1;
        const long rows_all = (long)sh.B * sh.H * sh.nq;
        float* ws_acc = S > 1 ? static_cast<float*>(ws) : nullptr;
        float2* ws_ml = S > 1 ? reinterpret_cast<float2*>(ws_acc + rows_all * S * sh.d) : nullptr;
        const long n_tiles = (sh.nq + kSpQ - 1) / kSpQ;
        note_path("readout: MFMA tiles of 128 queries over their union, %d split(s)", S);
        dim3 grid((unsigned)(n_tiles * S * sh.B * sh.H)), block(256);
#define FS_SPARSE_MFMA(D)                                                                         \
        hipLaunchKernelGGL((sparse_attn_mfma_kernel<D>), grid, block, lds, st,                    \
                           (const uint16_t*)q, sh.qs[0], sh.qs[1], sh.qs[2],                      \
                           (const uint16_t*)k, (const uint16_t*)v, sh.kvs[0], sh.kvs[1],          \
                           sh.kvs[2], sh.H, sh.B * sh.H, sh.nq, sh.C, idx, topk, scale_log2,      \
                           rms_eps,                                                               \
                           (uint16_t*)o_lr, sh.os[0], sh.os[1], sh.os[2], S, ws_acc, ws_ml,      \
                           (const uint16_t*)o_sr, alpha)
        if (sh.d == 64) FS_SPARSE_MFMA(64); else FS_SPARSE_MFMA(128);
#undef FS_SPARSE_MFMA
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || S <= 1) return err;
        return launch_split_merge(sh, S, ws_acc, ws_ml, true, rms_eps, o_lr, st, o_sr, alpha);
    }
    note_path("readout: row-wise, one wavefront per query (%s)",
              sh.C > kSpMaxCells ? "more than 32768 cells"
              : "the union bookkeeping exceeds 160 KiB of LDS");
    dim3 grid((unsigned)((sh.nq + 3) / 4), (unsigned)(sh.B * sh.H)), block(256);
#define FS_SPARSE(E, D)                                                                          \
    hipLaunchKernelGGL((sparse_attn_rowwise_kernel<E, D>), grid, block, 0, st,                   \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2],              \
                       (const typename E::storage*)k, (const typename E::storage*)v, sh.kvs[0],  \
                       sh.kvs[1], sh.kvs[2], sh.H, sh.nq, idx, topk, scale_log2, rms_eps,        \
                       (typename E::storage*)o_lr, sh.os[0], sh.os[1], sh.os[2],                 \
                       (const typename E::storage*)o_sr, alpha)
    if (sh.bf16) {
        if (sh.d == 64) FS_SPARSE(Bf16, 64); else FS_SPARSE(Bf16, 128);
    } else {
        if (sh.d == 64) FS_SPARSE(F32, 64); else FS_SPARSE(F32, 128);
    }
#undef FS_SPARSE
    return hipGetLastError();
}

}  // namespace fs
