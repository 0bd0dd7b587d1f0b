// stream.hip -- streaming FS-L state: append tokens, then attend from the state
// alone (FreeSolo summary, section 3.3 eqs. 5 and 8, and "Bounded memory" under
// Practical Implications).
//
// A step appends the next n_new tokens of every (batch, head) and evaluates
// eqs. 2-9 for the queries at those positions, reading only the fixed-size state
// of fs_stream.hpp.  One workgroup per (batch, head) updates the state:
//  1. the slots set aside by the previous step return to the free list;
//  2. the new keys and values go into the mirrored ring;
//  3. each cell that has become a candidate (its last token now precedes i - w)
//     is summarised from the ring with the batch summaries' wave arithmetic,
//     and eq. 8 is updated: the cell enters TopP if its (a_c, c) beats the
//     smallest entry (which it then evicts; being the newest cell it wins ties
//     on a_c), and it enters Recent_W, whose oldest cell leaves.  A kept cell is
//     copied into a free slot.  A cell that leaves both sets is set aside: its
//     slot is freed at the next step, because this step's earlier queries may
//     still read it.  TopP over [0, n + 1) is TopP over TopP(n) + {n}, so a cell
//     once dropped is never needed again;
//  4. after each cell (and before the first) the keep row of that candidate
//     count is written as pool slots in ascending cell order, when a query of
//     the step has that count.
// The queries then run: selection over their keep rows (stream_select_kernel),
// the window branch over the ring (the batch window kernel through a base
// pointer shifted so that position p addresses ring row p mod L, +L where it
// wraps), the readout over the pool (the batch readout with slots as cells) and
// eq. 2's combination.
#include "cell_summary.hpp"
#include "fs_device.hpp"
#include "fs_launch.hpp"
#include "fs_stream.hpp"

namespace fs {

namespace {

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

StreamLayout stream_layout(const StreamCfg& c)
{
    StreamLayout Ly;
    int L = 64;
    while (L < c.w + c.s + c.max_new) L <<= 1;
    Ly.L = L;
    Ly.M = c.W + c.P + (c.max_new + c.s - 1) / c.s + 2;
    Ly.R = (c.max_new + c.s - 1) / c.s + 2;
    Ly.keep_w = c.W + c.P;
    Ly.esize = c.bf16 ? 2 : 4;
    const size_t BH = (size_t)c.B * c.H;
    const size_t e = (size_t)Ly.esize;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = up256(off + bytes);
        return at;
    };
    Ly.hdr = take(BH * kHdrWords * 4);
    Ly.ring_k = take(BH * 2 * L * c.d * e);
    Ly.ring_v = take(BH * 2 * L * c.d * e);
    Ly.pool_k = take(BH * Ly.M * c.s * c.d * e);
    Ly.pool_v = take(BH * Ly.M * c.s * c.d * e);
    Ly.kbar = take(BH * Ly.M * c.d * 4);
    Ly.amax = take(BH * Ly.M * 4);
    Ly.cell = take(BH * Ly.M * 4);
    const size_t P1 = c.P > 0 ? c.P : 1, W1 = c.W > 0 ? c.W : 1;
    Ly.topp_a = take(BH * P1 * 4);
    Ly.topp_c = take(BH * P1 * 4);
    Ly.topp_s = take(BH * P1 * 4);
    Ly.recent = take(BH * W1 * 4);
    Ly.free_list = take(BH * Ly.M * 4);
    Ly.pend = take(BH * Ly.M * 4);
    Ly.keep = take(BH * Ly.R * Ly.keep_w * 4);
    Ly.keep_cnt = take(BH * Ly.R * 4);
    Ly.idx = take(BH * c.max_new * c.K * 4);
    Ly.osr = take(BH * c.max_new * c.d * e);
    Ly.olr = take(BH * c.max_new * c.d * e);
    Shape sh{};
    sh.B = c.B; sh.H = c.H; sh.d = c.d; sh.s = c.s; sh.w = c.w; sh.bf16 = c.bf16;
    sh.C = Ly.M; sh.N = Ly.M * c.s;
    size_t ws = 0, wws = 0;              // split workspaces, largest over n_new
    for (int nq = 1; nq <= c.max_new; ++nq) {
        sh.nq = nq;
        const size_t b = sparse_ws_bytes(sh), bw = window_workspace_bytes(sh);
        ws = b > ws ? b : ws;
        wws = bw > wws ? bw : wws;
    }
    Ly.table = take(wws);                // the window's table, then its split states
    Ly.table_bytes = wws;
    Ly.ws_bytes = ws;
    Ly.ws = take(ws);
    Ly.bytes = off;
    return Ly;
}

namespace {

struct StreamDev {
    int32_t* hdr;
    char* ring_k;
    char* ring_v;
    char* pool_k;
    char* pool_v;
    float* kbar;
    float* amax;
    int32_t* cell;
    float* topp_a;
    int32_t* topp_c;
    int32_t* topp_s;
    int32_t* recent;
    int32_t* free_list;
    int32_t* pend;
    int32_t* keep;
    int32_t* keep_cnt;
    int L, M, R, W, P, keep_w, s, w;
};

StreamDev stream_dev(const StreamCfg& c, const StreamLayout& Ly, void* state)
{
    char* b = static_cast<char*>(state);
    StreamDev sd;
    sd.hdr = reinterpret_cast<int32_t*>(b + Ly.hdr);
    sd.ring_k = b + Ly.ring_k;
    sd.ring_v = b + Ly.ring_v;
    sd.pool_k = b + Ly.pool_k;
    sd.pool_v = b + Ly.pool_v;
    sd.kbar = reinterpret_cast<float*>(b + Ly.kbar);
    sd.amax = reinterpret_cast<float*>(b + Ly.amax);
    sd.cell = reinterpret_cast<int32_t*>(b + Ly.cell);
    sd.topp_a = reinterpret_cast<float*>(b + Ly.topp_a);
    sd.topp_c = reinterpret_cast<int32_t*>(b + Ly.topp_c);
    sd.topp_s = reinterpret_cast<int32_t*>(b + Ly.topp_s);
    sd.recent = reinterpret_cast<int32_t*>(b + Ly.recent);
    sd.free_list = reinterpret_cast<int32_t*>(b + Ly.free_list);
    sd.pend = reinterpret_cast<int32_t*>(b + Ly.pend);
    sd.keep = reinterpret_cast<int32_t*>(b + Ly.keep);
    sd.keep_cnt = reinterpret_cast<int32_t*>(b + Ly.keep_cnt);
    sd.L = Ly.L; sd.M = Ly.M; sd.R = Ly.R; sd.W = c.W; sd.P = c.P;
    sd.keep_w = Ly.keep_w; sd.s = c.s; sd.w = c.w;
    return sd;
}

// Empty state: no tokens, no cells, every slot free.
__global__ __launch_bounds__(256) void stream_reset_kernel(StreamDev sd)
{
    const long bh = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < kHdrWords) sd.hdr[bh * kHdrWords + tid] = tid == kHdrFree ? sd.M : 0;
    for (int j = tid; j < sd.M; j += 256) {
        sd.free_list[bh * sd.M + j] = sd.M - 1 - j;
        sd.cell[bh * sd.M + j] = -1;
    }
}

constexpr int kNCB = 16;          // new cells summarised together (one wave each)
constexpr int kAppendWaves = 4;   // waves of the append workgroup

__device__ __forceinline__ int block_sum_int(int x, int* red)
{
    x = wave_sum_int(x);
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wv] = x;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ uint64_t block_min_u64(uint64_t x, uint64_t* red)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t y = __shfl_xor(x, m, kWave);
        x = y < x ? y : x;
    }
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wv] = x;
    __syncthreads();
    uint64_t r = red[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) r = red[j] < r ? red[j] : r;
    return r;
}

template <class E, int D>
__global__ __launch_bounds__(256) void stream_append_kernel(
    StreamDev sd, const typename E::storage* __restrict__ k_new,
    const typename E::storage* __restrict__ v_new, int n_new, int64_t pos0, int64_t n_start,
    int64_t n_end, int64_t n_row0)
{
    using T = typename E::storage;
    constexpr int EPV = E::kPer16B;   // elements per 16 bytes
    constexpr int CPR = D / EPV;      // 16-byte chunks per row
    extern __shared__ uint4 smem_raw[];
    const int P = sd.P, M = sd.M, W = sd.W, L = sd.L, s = sd.s;
    const int P1 = P > 0 ? P : 1, W1 = W > 0 ? W : 1;
    float* l_kbar = reinterpret_cast<float*>(smem_raw);                 // [kNCB][D], 16-byte aligned
    float* l_ta = l_kbar + kNCB * D;                                    // TopP a_c [P]
    int32_t* l_tc = reinterpret_cast<int32_t*>(l_ta + P1);              // TopP cell [P]
    int32_t* l_ts = l_tc + P1;                                          // TopP slot [P]
    int32_t* l_free = l_ts + P1;                                        // [M]
    int32_t* l_pend = l_free + M;                                       // [M]
    int32_t* l_intopp = l_pend + M;                                     // [M] slot in TopP
    int32_t* l_recent = l_intopp + M;                                   // [W]
    __shared__ float l_ab[kNCB];              // a_c of the batch's cells
    __shared__ int l_slot[kNCB];              // their slots (-1: not kept)
    __shared__ int red_i[4];
    __shared__ uint64_t red_u[4];
    __shared__ int s_pos;

    const int tid = threadIdx.x, wv = tid >> 6;
    const long bh = blockIdx.x;
    int32_t* hdr = sd.hdr + bh * kHdrWords;
    int tcount = hdr[kHdrTopP], fcount = hdr[kHdrFree];
    const int pcount0 = hdr[kHdrPend];
    int err = hdr[kHdrError];

    // ---- load the set structures; last step's set-aside slots become free
    for (int j = tid; j < tcount; j += 256) {
        l_ta[j] = sd.topp_a[bh * P1 + j];
        l_tc[j] = sd.topp_c[bh * P1 + j];
        l_ts[j] = sd.topp_s[bh * P1 + j];
    }
    for (int j = tid; j < fcount; j += 256) l_free[j] = sd.free_list[bh * M + j];
    for (int j = tid; j < pcount0; j += 256) l_free[fcount + j] = sd.pend[bh * M + j];
    fcount += pcount0;
    int pcount = 0;
    for (int j = tid; j < M; j += 256) l_intopp[j] = 0;
    for (int j = tid; j < W; j += 256) l_recent[j] = sd.recent[bh * W1 + j];
    __syncthreads();
    for (int j = tid; j < tcount; j += 256) l_intopp[l_ts[j]] = 1;

    // ---- new tokens into both copies of the ring
    T* rk = reinterpret_cast<T*>(sd.ring_k) + bh * (long)(2 * L) * D;
    T* rv = reinterpret_cast<T*>(sd.ring_v) + bh * (long)(2 * L) * D;
    const T* kn = k_new + bh * (long)n_new * D;
    const T* vn = v_new + bh * (long)n_new * D;
    for (int e = tid; e < n_new * CPR; e += 256) {
        const int t = e / CPR, ch = e % CPR;
        const int r = (int)((pos0 + t) & (L - 1));
        const uint4 kk = *reinterpret_cast<const uint4*>(kn + (long)t * D + ch * EPV);
        const uint4 vv = *reinterpret_cast<const uint4*>(vn + (long)t * D + ch * EPV);
        *reinterpret_cast<uint4*>(rk + (long)r * D + ch * EPV) = kk;
        *reinterpret_cast<uint4*>(rk + (long)(r + L) * D + ch * EPV) = kk;
        *reinterpret_cast<uint4*>(rv + (long)r * D + ch * EPV) = vv;
        *reinterpret_cast<uint4*>(rv + (long)(r + L) * D + ch * EPV) = vv;
    }
    __syncthreads();                    // ring rows visible to the whole workgroup

    // keep row of candidate count n: TopP cells below n - W, then the recent cells
    auto emit_row = [&](int64_t n) {
        const int rr = (int)(n - n_row0);
        int32_t* row = sd.keep + (bh * sd.R + rr) * (long)sd.keep_w;
        const int64_t lim = n - W;
        int npre = tcount;                    // W = 0: every TopP cell precedes n
        if (W > 0) {
            int below = 0;
            for (int j = tid; j < tcount; j += 256) below += l_tc[j] < lim;
            npre = block_sum_int(below, red_i);
        }
        const int nrec = (int)(n < W ? n : W);
        for (int j = tid; j < npre; j += 256) row[j] = l_ts[j];
        for (int j = tid; j < nrec; j += 256) row[npre + j] = l_recent[(int)((n - nrec + j) % W)];
        if (tid == 0) sd.keep_cnt[bh * sd.R + rr] = npre + nrec;
    };
    if (n_row0 == n_start) emit_row(n_start);

    bool stop = false;                        // block-uniform
    // TopP's smallest (a_c, c) and its position, valid until TopP changes
    bool min_ok = false;
    uint64_t kmin = 0;
    int kpos = 0;
    for (int64_t cb = n_start; cb < n_end && !stop; cb += kNCB) {
        const int nb = (int)(n_end - cb < kNCB ? n_end - cb : kNCB);
        // (a) summaries of the batch's cells, one wave per cell, from their 32 ring
        //     rows (contiguous thanks to the mirror)
        for (int j = wv; j < nb; j += kAppendWaves) {
            const int rbase = (int)(((cb + j) * s) & (L - 1));
            wave_cell_summary<E, D>(rk + (long)rbase * D, D, l_kbar + j * D, &l_ab[j]);
        }
        if (tid < kNCB) l_slot[tid] = -1;     // cells not reached keep no slot
        __syncthreads();
        for (int jc = 0; jc < nb && !stop; ++jc) {
            const int64_t c = cb + jc;
            const float a = l_ab[jc];
            // (b) eq. 8: does (a, c) beat TopP's smallest (a_c, c)?
            bool enter = tcount < P;
            int ev = -1;
            if (!enter && P > 0) {
                if (!min_ok) {                // block-uniform
                    uint64_t mine = ~0ull;
                    for (int j = tid; j < tcount; j += 256) {
                        const uint64_t kk =
                            ((uint64_t)__float_as_uint(l_ta[j]) << 32) | (uint32_t)l_tc[j];
                        mine = kk < mine ? kk : mine;
                    }
                    kmin = block_min_u64(mine, red_u);
                    const int cmin = (int)(uint32_t)kmin;
                    for (int j = tid; j < tcount; j += 256)
                        if (l_tc[j] == cmin) s_pos = j;
                    __syncthreads();
                    kpos = s_pos;
                    min_ok = true;
                }
                // a_c >= 0, so its bit pattern orders like its value; c is newer than
                // every stored cell and wins a tie on a_c
                enter = __float_as_uint(a) >= (uint32_t)(kmin >> 32);
                ev = enter ? kpos : -1;
            }
            if (enter) min_ok = false;        // TopP changes below
            const int ce = ev >= 0 ? l_tc[ev] : -1, se = ev >= 0 ? l_ts[ev] : -1;
            const int64_t cr = (W > 0 && c - W >= 0) ? c - W : -1;   // leaves Recent_W
            const int sr = cr >= 0 ? l_recent[(int)(cr % W)] : -1;
            const bool retained = enter || W > 0;
            if (retained && fcount == 0) {       // cannot happen with M slots; flagged, not faulted
                err = 1;
                stop = true;
                break;
            }
            const int slot = retained ? l_free[fcount - 1] : -1;
            if (retained) --fcount;
            // set aside: the evicted cell unless Recent_W (cells c-W+1 .. c) keeps it, and
            // the cell leaving Recent_W unless TopP keeps it (counted once if both)
            const bool drop_e = ev >= 0 && ce <= c - W;
            const bool drop_r = cr >= 0 && cr != ce && !l_intopp[sr];
            __syncthreads();                     // every thread has read the entries it needs

            // (c) TopP update, in ascending cell order: drop entry ev, append c
            if (enter) {
                if (ev >= 0) {
                    float va[4];
                    int32_t vc[4], vs[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int j = tid + 256 * u;
                        if (j > ev && j < tcount) { va[u] = l_ta[j]; vc[u] = l_tc[j]; vs[u] = l_ts[j]; }
                    }
                    __syncthreads();
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int j = tid + 256 * u;
                        if (j > ev && j < tcount) { l_ta[j - 1] = va[u]; l_tc[j - 1] = vc[u]; l_ts[j - 1] = vs[u]; }
                    }
                    --tcount;
                }
                if (tid == 0) {                  // index tcount is not among the shifted ones
                    l_ta[tcount] = a;
                    l_tc[tcount] = (int32_t)c;
                    l_ts[tcount] = slot;
                }
                ++tcount;
            }
            // (d) set-aside list, TopP membership, Recent_W
            if (tid == 0) {
                if (ev >= 0) l_intopp[se] = 0;
                if (enter) l_intopp[slot] = 1;
                if (drop_e) l_pend[pcount] = se;
                if (drop_r) l_pend[pcount + drop_e] = sr;
                if (W > 0) l_recent[(int)(c % W)] = slot;
            }
            pcount += (int)drop_e + (int)drop_r;
            if (tid == 0) l_slot[jc] = retained ? slot : -1;
            __syncthreads();
            if (c + 1 >= n_row0) emit_row(c + 1);
            __syncthreads();
        }
        // (e) the batch's kept cells are copied into their slots with their summaries
        for (int e = tid; e < nb * s * CPR; e += 256) {
            const int j = e / (s * CPR), t = (e / CPR) % s, ch = e % CPR;
            const int slot = l_slot[j];
            if (slot < 0) continue;
            const int rbase = (int)(((cb + j) * s) & (L - 1));
            T* pk = reinterpret_cast<T*>(sd.pool_k) + (bh * M + slot) * (long)s * D;
            T* pv = reinterpret_cast<T*>(sd.pool_v) + (bh * M + slot) * (long)s * D;
            const long src = (long)(rbase + t) * D + ch * EPV;
            *reinterpret_cast<uint4*>(pk + (long)t * D + ch * EPV) =
                *reinterpret_cast<const uint4*>(rk + src);
            *reinterpret_cast<uint4*>(pv + (long)t * D + ch * EPV) =
                *reinterpret_cast<const uint4*>(rv + src);
        }
        for (int e = tid; e < nb * D; e += 256) {
            const int slot = l_slot[e / D];
            if (slot >= 0) sd.kbar[(bh * M + slot) * (long)D + e % D] = l_kbar[e];
        }
        for (int j = tid; j < nb; j += 256) {
            if (l_slot[j] >= 0) {
                sd.amax[bh * M + l_slot[j]] = l_ab[j];
                sd.cell[bh * M + l_slot[j]] = (int32_t)(cb + j);
            }
        }
        __syncthreads();                      // l_kbar, l_ab and l_slot are reused
    }

    // ---- write the set structures back
    for (int j = tid; j < tcount; j += 256) {
        sd.topp_a[bh * P1 + j] = l_ta[j];
        sd.topp_c[bh * P1 + j] = l_tc[j];
        sd.topp_s[bh * P1 + j] = l_ts[j];
    }
    for (int j = tid; j < fcount; j += 256) sd.free_list[bh * M + j] = l_free[j];
    for (int j = tid; j < pcount; j += 256) sd.pend[bh * M + j] = l_pend[j];
    for (int j = tid; j < W; j += 256) sd.recent[bh * W1 + j] = l_recent[j];
    if (tid == 0) {
        hdr[kHdrTokens] = (int32_t)(pos0 + n_new);
        hdr[kHdrCells] = (int32_t)n_end;
        hdr[kHdrTopP] = tcount;
        hdr[kHdrFree] = fcount;
        hdr[kHdrPend] = pcount;
        hdr[kHdrError] = err;
    }
}

}  // namespace

hipError_t launch_stream_reset(const StreamCfg& c, const StreamLayout& Ly, void* state,
                               hipStream_t st)
{
    const StreamDev sd = stream_dev(c, Ly, state);
    hipLaunchKernelGGL(stream_reset_kernel, dim3((unsigned)(c.B * c.H)), dim3(256), 0, st, sd);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    Shape sh{};
    sh.d = c.d; sh.w = c.w;
    return launch_rope_table(sh, c.rope_base, static_cast<char*>(state) + Ly.table, st);
}

hipError_t launch_stream_step(const StreamCfg& c, const StreamLayout& Ly, void* state,
                              int64_t pos0, int n_new, const void* q, const void* k,
                              const void* v, const float* alpha, const float* lambda,
                              const float* sigma, void* o, int32_t* idx_cell, hipStream_t st)
{
    if (n_new == 0) return hipSuccess;
    const StreamDev sd = stream_dev(c, Ly, state);
    char* base = static_cast<char*>(state);
    auto ncand = [&](int64_t i) -> int64_t { return i < c.w ? 0 : (i - c.w) / c.s; };
    const int64_t n_start = pos0 == 0 ? 0 : ncand(pos0 - 1);
    const int64_t n_row0 = ncand(pos0), n_end = ncand(pos0 + n_new - 1);

    // 1. state update
    const int P1 = c.P > 0 ? c.P : 1, W1 = c.W > 0 ? c.W : 1;
    const size_t lds = (size_t)kNCB * c.d * 4 + (size_t)3 * P1 * 4 + (size_t)3 * Ly.M * 4 +
                       (size_t)W1 * 4;
#define FS_APPEND(E, D)                                                                          \
    hipLaunchKernelGGL((stream_append_kernel<E, D>), dim3((unsigned)(c.B * c.H)), dim3(256), lds, \
                       st, sd, (const typename E::storage*)k, (const typename E::storage*)v,      \
                       n_new, pos0, n_start, n_end, n_row0)
    if (c.bf16) {
        if (c.d == 64) FS_APPEND(Bf16, 64); else FS_APPEND(Bf16, 128);
    } else {
        if (c.d == 64) FS_APPEND(F32, 64); else FS_APPEND(F32, 128);
    }
#undef FS_APPEND
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    // q, o: contiguous [B][H][n_new][d]
    const int64_t io[3] = {(int64_t)c.H * n_new * c.d, (int64_t)n_new * c.d, c.d};
    int32_t* idx_slot = reinterpret_cast<int32_t*>(base + Ly.idx);
    // 2. eq. 7 selection over the keep rows
    err = launch_stream_select(c.B, c.H, c.d, c.bf16 != 0, q, io, sd.kbar, sd.amax, sd.cell, Ly.M,
                               lambda, sigma, n_new, pos0, c.w, c.s, sd.keep, sd.keep_cnt,
                               Ly.keep_w, n_row0, Ly.R, c.K, idx_slot, idx_cell, nullptr, st);
    if (err != hipSuccess) return err;

    Shape sh{};
    sh.B = c.B; sh.H = c.H; sh.d = c.d; sh.s = c.s; sh.w = c.w; sh.bf16 = c.bf16;
    sh.nq = n_new;
    for (int t = 0; t < 3; ++t) sh.qs[t] = sh.os[t] = io[t];
    // 3. window branch over the ring: position p of [lo, pos0 + n_new) is row
    //    (lo mod L) + (p - lo) of the doubled ring, lo = max(0, pos0 - w)
    const int64_t lo = pos0 - c.w > 0 ? pos0 - c.w : 0;
    const int64_t shift = (lo & (Ly.L - 1)) - lo;          // rows, <= 0
    sh.q_pos0 = (int)pos0;
    sh.N = (int)(pos0 + n_new);
    sh.C = sh.N / c.s;
    sh.kvs[0] = (int64_t)c.H * 2 * Ly.L * c.d;
    sh.kvs[1] = (int64_t)2 * Ly.L * c.d;
    sh.kvs[2] = c.d;
    const char* kwin = sd.ring_k + shift * c.d * Ly.esize;
    const char* vwin = sd.ring_v + shift * c.d * Ly.esize;
    err = launch_window(sh, q, kwin, vwin, c.rope_base, base + Ly.table, base + Ly.osr, st,
                        true, Ly.table_bytes);               // tabulated at the reset
    if (err != hipSuccess) return err;
    // 4. readout over the pool: slot u's tokens are rows u s .. u s + s - 1
    sh.q_pos0 = 0;
    sh.C = Ly.M;
    sh.N = Ly.M * c.s;
    sh.kvs[0] = (int64_t)c.H * Ly.M * c.s * c.d;
    sh.kvs[1] = (int64_t)Ly.M * c.s * c.d;
    sh.kvs[2] = c.d;
    // 5. eq. 2 in the readout's epilogue: o = o_sr + alpha_h o_lr
    return launch_sparse(sh, q, sd.pool_k, sd.pool_v, idx_slot, c.K, c.rms_eps,
                         Ly.ws_bytes ? base + Ly.ws : nullptr, o, st, base + Ly.osr, alpha);
}

}  // namespace fs
