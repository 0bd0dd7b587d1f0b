// select.hip -- cell scoring and per-query top-K (FreeSolo summary, section 3.3,
// eq. 7 with lambda_h = 0; the selected set S_i of eq. 9).
//
// One wavefront per query row.  The unrotated query is staged in LDS; each lane
// scores candidate cells c (from the keep row of the query's candidate count,
// or every c < n_i without pruning) as the fp32 dot q . kbar_c.  Ranking uses
// the unscaled dot (1/sqrt(d) > 0 does not change the order and must not merge
// neighbouring scores); the reported score is dot / sqrt(d).  The K-th largest
// key is found exactly by a bitwise search with ballot counts, ties at the
// threshold go to the larger cell, and the chosen cells are written ascending.
//
// bf16 storage (candidate lists up to 640 cells): MFMA kernel.  A workgroup
// owns 64 consecutive queries (4 wavefronts x 16); they span at most three
// candidate counts, so their candidates are the union of at most three keep
// rows (or the prefix [0, n) without pruning), built in LDS with a bitmap.
// kbar rows of the union are staged 64 at a time, each fp32 value split into
// three bf16 parts hi + mid + lo (24 significant bits); q is exact in bf16, so
// three exact-product MFMAs with fp32 accumulation give fp32-accurate scores.
// The scores go to LDS as order-preserving keys; each query's row is then
// loaded into 4 consecutive lanes (a DPP quad; all 16 queries of a wave at
// once), the K-th largest key is found by the same bitwise search with quad
// DPP sums, and the chosen cells are written in slot order from one exclusive
// prefix over the quad.
#include "fs_device.hpp"
#include "fs_launch.hpp"
#include "mfma_tile.hpp"

namespace fs {

constexpr int kSelWaves = 4;

__device__ __forceinline__ float key_to_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <class E, int D>
__global__ __launch_bounds__(kSelWaves * kWave) void select_topk_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ kbar, int H, int C, int nq, int q_pos0, int window, int cell,
    const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_count, int keep_w,
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
        s_key[j] = float_key(dot);
    }
    __syncthreads();
    if (!active) return;

    const int kq = n_cand < topk ? n_cand : topk;
    uint32_t thr = 0;
    if (kq > 0) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t t = thr | (1u << bit);
            int cnt = 0;
            for (int j = lane; j < n_cand; j += kWave) cnt += s_key[j] >= t;
            if (wave_sum_int(cnt) >= kq) thr = t;
        }
    }
    int n_gt = 0, n_eq = 0;
    for (int j = lane; j < n_cand; j += kWave) {
        n_gt += s_key[j] > thr;
        n_eq += s_key[j] == thr;
    }
    n_gt = wave_sum_int(n_gt);
    n_eq = wave_sum_int(n_eq);
    const int need_eq = kq - n_gt;

    int32_t* out_i = idx + (bh * nq + row) * (long)topk;
    float* out_s = score ? score + (bh * nq + row) * (long)topk : nullptr;
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
        if (kept) {
            const int pos = written + lanes_below(mk);
            out_i[pos] = cand ? cand[j] : j;
            if (out_s) out_s[pos] = key_to_float(kj) * inv_sqrt_d;
        }
        written += __popcll(mk);
        eq_seen += __popcll(me);
    }
    for (int t = kq + lane; t < topk; t += kWave) {
        out_i[t] = -1;
        if (out_s) out_s[t] = 0.f;
    }
}


namespace {

constexpr int kSelChunk = 32;        // union cells staged per chunk (two 16-cell MFMA blocks)
constexpr int kSelMaxCells = 32768;
constexpr int kSelLdsMax = 160 * 1024;
constexpr int kSelMaxKeysPerLane = 132;  // quad layout: union of at most 528 cells per block

struct SelLayout {
    int nwords, u_cap, waves, keep_w;
    size_t off_keys, off_bitmap, off_rank, off_ulist, off_vmask, off_krows, bytes;
};

// LDS carve-up: kbar chunk split in 3 bf16 parts | keys [16*waves][u_cap] |
// bitmap | rank | union list | row-membership masks | copy of the keep rows.
template <int D>
__host__ __device__ inline SelLayout sel_layout(int n_hi, int u_cap, int waves, int keep_w)
{
    SelLayout L;
    L.nwords = (n_hi + 31) / 32;
    L.u_cap = u_cap;
    L.waves = waves;
    L.keep_w = keep_w;
    auto up16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
    size_t off = (size_t)3 * kSelChunk * mf::KPitch<D>::value * 2;
    L.off_keys = off;
    off = up16(off + (size_t)16 * waves * u_cap * 4);
    L.off_bitmap = off;
    off = up16(off + (size_t)L.nwords * 4);
    L.off_rank = off;
    off = up16(off + (size_t)L.nwords * 2);
    L.off_ulist = off;
    off = up16(off + (size_t)u_cap * 2);
    L.off_vmask = off;
    off = up16(off + (size_t)u_cap * 4);
    L.off_krows = off;
    off = up16(off + (size_t)3 * keep_w * 2);
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

}  // namespace

template <int D, int KPQ>
__global__ __launch_bounds__(256) void select_topk_mfma_kernel(   // 256 threads exactly
    const uint16_t* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ kbar, int H, int BH, int C, int nq, int q_pos0, int window,
    int cell, const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_count,
    int keep_w, int n_lo, int n_rows, int topk, int n_hi_all, int u_cap, float inv_sqrt_d,
    int32_t* __restrict__ idx, float* __restrict__ score)
{
    using namespace mf;
    constexpr int KP = KPitch<D>::value;
    constexpr int KS = D / 32;
    const int waves = blockDim.x >> 6, tq = 16 * waves;
    extern __shared__ uint4 smem_raw[];
    const SelLayout L = sel_layout<D>(n_hi_all, u_cap, waves, keep ? keep_w : 0);
    char* base = reinterpret_cast<char*>(smem_raw);
    uint16_t* kbs = reinterpret_cast<uint16_t*>(base);      // [3][kSelChunk][KP]
    uint32_t* keys = reinterpret_cast<uint32_t*>(base + L.off_keys);
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
    const long t0 = tb.tile * tq;
    const int n_rows_blk = nq - t0 < tq ? (int)(nq - t0) : tq;
    const int n_a = n_candidates((long)q_pos0 + t0, window, cell, C);
    const int n_b = n_candidates((long)q_pos0 + t0 + n_rows_blk - 1, window, cell, C);

    // ---- union of the candidate sets of the block's queries --------------
    int n_union;
    if (keep != nullptr) {
        const int nw = (n_b + 31) >> 5;
        // the (at most three) keep rows, copied to LDS with all loads in flight together
        const int r_first = n_a > 1 ? n_a : 1;            // rows of n = 0 are empty
        const int n_kr = n_b >= r_first ? n_b - r_first + 1 : 0;
        int kcnt[3];
#pragma unroll
        for (int j = 0; j < 3; ++j)
            kcnt[j] = j < n_kr ? keep_count[bh * n_rows + (r_first + j - n_lo)] : 0;
        for (int e0 = 0; e0 < 3 * keep_w; e0 += 4 * 256) {
            int vals[4];
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
                const int e = e0 + u4 * 256 + tid;
                const int j = e / keep_w, x = e - j * keep_w;
                const int cnt = j == 0 ? kcnt[0] : j == 1 ? kcnt[1] : kcnt[2];
                vals[u4] = (j < 3 && x < cnt)
                               ? keep[(bh * n_rows + (r_first + j - n_lo)) * keep_w + x] : -1;
            }
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
                const int e = e0 + u4 * 256 + tid;
                if (e < 3 * keep_w) krows[e] = (uint16_t)(vals[u4] < 0 ? 0xFFFF : vals[u4]);
            }
        }
        for (int wd = tid; wd < nw; wd += 256) bitmap[wd] = 0u;
        __syncthreads();
        for (int e = tid; e < 3 * keep_w; e += 256) {
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
        for (int e = tid; e < 3 * keep_w; e += 256) {
            const int c = krows[e];
            if (c != 0xFFFF) {
                const int sl = rank[c >> 5] + __popc(bitmap[c >> 5] & ((1u << (c & 31)) - 1u));
                atomicOr(&vmask[sl], 1u << (r_first + e / keep_w - n_a));
            }
        }
    } else {
        n_union = n_b;   // candidates are the prefix [0, n_i); slot == cell
    }

    // ---- the wave's 16 queries as B operands --------------------------------
    const int qr = 16 * wv + n;                 // this lane's query row in the block
    const bool q_ok = qr < n_rows_blk;
    const int n_q = q_ok ? n_candidates((long)q_pos0 + t0 + qr, window, cell, C) : 0;
    bf16x8 qf[KS];
    {
        const uint16_t* qrow = q + b * qs0 + h * qs1 + (t0 + (q_ok ? qr : 0)) * qs2;
#pragma unroll
        for (int t = 0; t < KS; ++t)
            qf[t] = as_bf16x8(q_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * g)
                                   : make_uint4(0, 0, 0, 0));
    }

    // ---- scores S^T = Kbar Q^T over the union, kSelChunk cells per step -------
    // The next chunk's kbar rows are loaded into registers while the current
    // chunk's MFMAs run.
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
    __syncthreads();                         // ulist complete
    load_chunk(0);
    for (int c0 = 0; c0 < n_union; c0 += kSelChunk) {
        __syncthreads();                     // previous chunk's MFMA reads are done
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int f = tid + 256 * it;
            const int cl = f / (D / 4), d4 = (f % (D / 4)) * 4;
            const float r[4] = {pre[it].x, pre[it].y, pre[it].z, pre[it].w};
            // x = hi + mid + lo exactly: each residual has at most 16 (then 8)
            // significant bits, so the fp32 subtractions are exact.
            uint32_t part[3][2];
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                float a0 = r[e], a1 = r[e + 1];
                const uint32_t h = cvt_pk_bf16(a0, a1);
                a0 -= __uint_as_float(h << 16);
                a1 -= __uint_as_float(h & 0xFFFF0000u);
                const uint32_t m = cvt_pk_bf16(a0, a1);
                a0 -= __uint_as_float(m << 16);
                a1 -= __uint_as_float(m & 0xFFFF0000u);
                part[0][e / 2] = h;
                part[1][e / 2] = m;
                part[2][e / 2] = cvt_pk_bf16(a0, a1);
            }
#pragma unroll
            for (int pp = 0; pp < 3; ++pp)
                *reinterpret_cast<uint2*>(kbs + (pp * kSelChunk + cl) * KP + d4) =
                    make_uint2(part[pp][0], part[pp][1]);
        }
        __syncthreads();
        if (c0 + kSelChunk < n_union) load_chunk(c0 + kSelChunk);
#pragma unroll
        for (int bb = 0; bb < kSelChunk / 16; ++bb) {
            const int slot0 = c0 + 16 * bb;
            if (slot0 >= n_union) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KS; ++t) {
#pragma unroll
                for (int pp = 0; pp < 3; ++pp) {
                    const bf16x8 a = as_bf16x8(
                        lds_load16(kbs + (pp * kSelChunk + 16 * bb + n) * KP + 32 * t + 8 * g));
                    acc = mfma(a, qf[t], acc);
                }
            }
            uint32_t kk[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = slot0 + 4 * g + r;
                bool ok = slot < n_union && n_q > 0;
                if (ok) ok = keep ? ((vmask[slot] >> (n_q - n_a)) & 1u) != 0u : slot < n_q;
                kk[r] = ok ? float_key(acc[r]) : 0u;
            }
            uint32_t* krow = keys + (size_t)qr * u_cap + slot0 + 4 * g;
            if (slot0 + 4 * g + 3 < u_cap) {   // u_cap is a multiple of 16
                *reinterpret_cast<uint4*>(krow) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (slot0 + 4 * g + r < u_cap) krow[r] = kk[r];
            }
        }
    }
    __syncthreads();

    // ---- per query: exact top-K, written in ascending slot (= cell) order ----
    // Quad layout: lanes 4j .. 4j+3 of wave w hold query 16w + j; lane 4j+sub
    // holds the contiguous slots [sub*kpq, (sub+1)*kpq) of that query's keys.
    {
        const int qj = lane >> 2, sub = lane & 3;
        const int row_b = 16 * wv + qj;
        const bool row_ok = row_b < n_rows_blk;
        const uint32_t* krow = keys + (size_t)row_b * u_cap + sub * KPQ;
        const int slot0 = sub * KPQ;
        uint32_t kv[KPQ];           // keys past the union are 0 and never counted
#pragma unroll
        for (int e = 0; e < KPQ; e += 4) {
            const uint4 w4 = *reinterpret_cast<const uint4*>(krow + e);
            kv[e] = slot0 + e < n_union ? w4.x : 0u;
            kv[e + 1] = slot0 + e + 1 < n_union ? w4.y : 0u;
            kv[e + 2] = slot0 + e + 2 < n_union ? w4.z : 0u;
            kv[e + 3] = slot0 + e + 3 < n_union ? w4.w : 0u;
        }
        int nv = 0;
#pragma unroll
        for (int e = 0; e < KPQ; ++e) nv += kv[e] != 0u;
        nv = quad_sum(nv);
        const int kq = nv < topk ? nv : topk;
        // kq-th largest key: the largest thr with #{key >= thr} >= kq
        uint32_t thr = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int c0 = 0, c1 = 0;                   // two chains: shorter dependency
#pragma unroll
            for (int e = 0; e < KPQ; e += 2) {
                c0 += kv[e] >= cand;
                c1 += kv[e + 1] >= cand;
            }
            if (quad_sum(c0 + c1) >= kq) thr = cand;
        }
        // thr >= 1 whenever kq > 0, so "key >= thr" and "key > thr" imply a valid key
        int ge = 0, gt = 0;
#pragma unroll
        for (int e = 0; e < KPQ; ++e) {
            ge += kv[e] >= thr;
            gt += kv[e] > thr;
        }
        const int eq = ge - gt;
        const int n_gt = quad_sum(gt), n_eq = quad_sum(eq);
        const int need_eq = kq - n_gt;            // equal keys kept: those in the largest slots
        const long orow = bh * nq + t0 + (row_ok ? row_b : 0);
        int32_t* out_i = idx + orow * topk;
        float* out_s = score ? score + orow * topk : nullptr;
        auto emit = [&](int p, uint32_t k, int j) {
            out_i[p] = keep ? ulist[j] : j;
            if (out_s) {
                const float dot = __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
                out_s[p] = dot * inv_sqrt_d;
            }
        };
        uint32_t thr_o = thr;
        asm volatile("" : "+v"(thr_o));           // fresh compares below, not kept masks
        if (n_eq == need_eq) {
            // no tie across the boundary: exactly the keys >= thr
            int pos = quad_excl_prefix(ge);
            if (row_ok && kq > 0) {
#pragma unroll
                for (int e = 0; e < KPQ; ++e) {
                    if (kv[e] >= thr_o) emit(pos++, kv[e], slot0 + e);
                }
            }
        } else {
            // ties at the threshold: keep the need_eq equal keys with the largest slots
            int eq_rank = quad_excl_prefix(eq);
            int kept_here = 0;
#pragma unroll
            for (int e = 0; e < KPQ; ++e) {
                const bool is_eq = kv[e] == thr_o;
                kept_here += kv[e] > thr_o || (is_eq && eq_rank >= n_eq - need_eq);
                eq_rank += is_eq;
            }
            int pos = quad_excl_prefix(kept_here);
            eq_rank = quad_excl_prefix(eq);
            if (row_ok && kq > 0) {
#pragma unroll
                for (int e = 0; e < KPQ; ++e) {
                    const bool is_eq = kv[e] == thr_o;
                    const bool kept = kv[e] > thr_o || (is_eq && eq_rank >= n_eq - need_eq);
                    eq_rank += is_eq;
                    if (kept) emit(pos++, kv[e], slot0 + e);
                }
            }
        }
        if (row_ok) {
            for (int t = kq + sub; t < topk; t += 4) {
                out_i[t] = -1;
                if (out_s) out_s[t] = 0.f;
            }
        }
    }
}

hipError_t launch_select(const Shape& sh, const void* q, const float* kbar, const int32_t* keep,
                         const int32_t* keep_count, int keep_w, int n_lo, int n_rows, int topk,
                         int32_t* idx, float* score, hipStream_t st)
{
    if (sh.nq == 0) return hipSuccess;
    // Largest candidate list: the keep width, or every cell below the last query's n.
    int n_hi = 0;
    {
        long i = (long)sh.q_pos0 + sh.nq - 1;
        if (i >= sh.w) n_hi = (int)((i - sh.w) / sh.s);
        if (n_hi > sh.C) n_hi = sh.C;
    }
    // MFMA path: bf16 storage; the block's scores must fit in LDS.
    {
        const int u_cap = keep ? (keep_w + 3 < n_hi ? keep_w + 3 : n_hi) : n_hi;
        const int uc = ((u_cap > 0 ? u_cap : 1) + 15) & ~15;     // rows 16-key aligned
        const int waves = 4;
        const int kw = keep ? keep_w : 0;
        const size_t lds = sh.d == 64 ? sel_layout<64>(n_hi, uc, waves, kw).bytes
                                      : sel_layout<128>(n_hi, uc, waves, kw).bytes;
        if (sh.bf16 && lds <= (size_t)kSelLdsMax && sh.C <= kSelMaxCells &&
            uc <= 4 * kSelMaxKeysPerLane) {
            const int tq = 16 * waves;
            dim3 grid((unsigned)((sh.nq + tq - 1) / tq * sh.B * sh.H));
            const float inv_sqrt_d = 1.0f / sqrtf((float)sh.d);
            const int kpq_need = uc / 4;          // multiple of 4
#define FS_SELECT_MFMA(D, KPL)                                                                  \
            hipLaunchKernelGGL((select_topk_mfma_kernel<D, KPL>), grid, dim3(64 * waves), lds,    \
                               st, (const uint16_t*)q, sh.qs[0], sh.qs[1], sh.qs[2], kbar, sh.H, \
                               sh.B * sh.H, sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep,            \
                               keep_count, keep_w,                                               \
                               n_lo, n_rows, topk, n_hi, uc, inv_sqrt_d, idx, score)
#define FS_SELECT_KPL(D)                                                                        \
            if (kpq_need <= 8) FS_SELECT_MFMA(D, 8);                                            \
            else if (kpq_need <= 16) FS_SELECT_MFMA(D, 16);                                     \
            else if (kpq_need <= 36) FS_SELECT_MFMA(D, 36);                                     \
            else if (kpq_need <= 68) FS_SELECT_MFMA(D, 68);                                     \
            else FS_SELECT_MFMA(D, 132);
            if (sh.d == 64) { FS_SELECT_KPL(64) } else { FS_SELECT_KPL(128) }
#undef FS_SELECT_KPL
#undef FS_SELECT_MFMA
            return hipGetLastError();
        }
    }
    const int cap = keep ? keep_w : (n_hi > 0 ? n_hi : 1);
    // As many waves (query rows) per block as fit in 64 KiB of LDS.
    int waves = kSelWaves;
    while (waves > 1 && (size_t)waves * (sh.d + cap) * sizeof(uint32_t) > 65536) waves >>= 1;
    const size_t lds = (size_t)waves * (sh.d + cap) * sizeof(uint32_t);
    if (lds > 65536) return hipErrorInvalidValue;
    dim3 grid((unsigned)((sh.nq + waves - 1) / waves), (unsigned)(sh.B * sh.H));
    dim3 block(waves * kWave);
    const float inv_sqrt_d = 1.0f / sqrtf((float)sh.d);
#define FS_SELECT(E, D)                                                                        \
    hipLaunchKernelGGL((select_topk_kernel<E, D>), grid, block, lds, st,                       \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2], kbar, sh.H, \
                       sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep, keep_count, keep_w, n_lo,      \
                       n_rows, topk, cap, inv_sqrt_d, idx, score)
    if (sh.bf16) {
        if (sh.d == 64) FS_SELECT(Bf16, 64); else FS_SELECT(Bf16, 128);
    } else {
        if (sh.d == 64) FS_SELECT(F32, 64); else FS_SELECT(F32, 128);
    }
#undef FS_SELECT
    return hipGetLastError();
}

}  // namespace fs
