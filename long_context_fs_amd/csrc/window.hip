// window.hip -- local RoPE branch (FreeSolo summary, section 3.2, eqs. 3-4).
//
// Eq. 3's right-hand side, q_i . R(j - i) k_j, depends on positions only through
// j - i.  The kernels therefore rotate by relative offsets taken from a cos/sin
// table built in fp64 (then rounded to fp32) for offsets -w-128 .. 127.  No
// absolute angle i * theta is ever formed in fp32, so accuracy does not decay
// at 256k positions.
//
// bf16 storage: flash-style MFMA kernel.  A workgroup owns 128 consecutive
// queries (4 wavefronts x 32) and walks the key range [i0 - w, i0 + 127] in
// tiles of 64 keys.  Each tile is staged in LDS once for the four waves: K
// rotated by R(j - i0) and rounded to fp16, V transposed (key-permuted, see
// mfma_tile.hpp).  Queries are rotated by R(i - i0) once and kept in registers
// as MFMA B operands.  The rotated q and k are no longer the exact bf16 inputs,
// so they are carried in fp16 (11-bit mantissa: 8x less rounding than bf16 at
// the same MFMA rate); this requires rotated elements below 65504 in magnitude.
// Per tile a wave computes S^T = K Q^T (16x16x32 fp16 MFMA, fp32 accumulate),
// masks to max(0, i-w) <= j <= i, runs the online
// softmax in fp32 (exp2 with log2(e)/sqrt(d) folded into the scale), and
// accumulates O^T += V^T P^T with P rounded to bf16.  The next tile's global
// loads are issued before the current tile's MFMAs (register double buffer).
// When the query tiles alone would leave the chip idle (decode), a tile's key
// range is split over workgroups whose partial (max, sum, O) states the
// readout's merge kernel combines.
// f32 storage: one wavefront per query, all in fp32.
#include "fs_device.hpp"
#include "fs_launch.hpp"
#include "mfma_tile.hpp"

namespace fs {

constexpr int kTableSlack = 128;   // table rows cover offsets [-w - slack, slack)

size_t rope_table_bytes(const Shape& sh)
{
    return (size_t)(sh.w + 2 * kTableSlack) * (sh.d / 2) * sizeof(float2);
}

// table[(delta + w + slack) * (d/2) + k] = (cos, sin)(delta * base^(-2k/d)), in fp64.
__global__ void rope_table_kernel(float2* __restrict__ table, int rows, int half, int w,
                                  double log_base)
{
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long)rows * half) return;
    const int r = (int)(t / half), k = (int)(t % half);
    const double theta = exp(-2.0 * (double)k / (double)(2 * half) * log_base);
    const double ang = (double)(r - w - kTableSlack) * theta;
    double s, c;
    sincos(ang, &s, &c);
    table[t] = make_float2((float)c, (float)s);
}

// One wavefront per query row; lanes take 64 keys at a time.
template <class E, int D>
__global__ __launch_bounds__(256) void window_attn_rowwise_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const typename E::storage* __restrict__ k, const typename E::storage* __restrict__ v,
    int64_t kvs0, int64_t kvs1, int64_t kvs2, int H, int nq, int q_pos0, int w,
    const float2* __restrict__ table, float scale_log2, typename E::storage* __restrict__ o,
    int64_t os0, int64_t os1, int64_t os2)
{
    constexpr int EPL = E::kPer16B;
    constexpr int R = D / kWave;       // output elements per lane
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

    const long i = (long)q_pos0 + row;
    const long lo = i - w > 0 ? i - w : 0;
    const typename E::storage* kh = k + b * kvs0 + h * kvs1;
    const typename E::storage* vh = v + b * kvs0 + h * kvs1;
    const float* qv = s_q[wv];

    float m = -INFINITY, l = 0.f, acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    for (long j0 = lo; j0 <= i; j0 += kWave) {
        const long j = j0 + lane;
        const bool valid = j <= i;
        float s = -INFINITY;
        if (valid) {
            const float2* rot = table + (long)(j - i + w + kTableSlack) * (D / 2);
            const typename E::storage* kr = kh + j * kvs2;
            float dot = 0.f;
            for (int e0 = 0; e0 < D; e0 += EPL) {
                float x[EPL];
                load16<E>(kr + e0, x);
#pragma unroll
                for (int p = 0; p < EPL / 2; ++p) {
                    const float2 cs = rot[e0 / 2 + p];
                    const float kx = x[2 * p] * cs.x - x[2 * p + 1] * cs.y;
                    const float ky = x[2 * p] * cs.y + x[2 * p + 1] * cs.x;
                    dot = fmaf(qv[e0 + 2 * p], kx, dot);
                    dot = fmaf(qv[e0 + 2 * p + 1], ky, dot);
                }
            }
            s = dot * scale_log2;
        }
        const float m_new = fmaxf(m, wave_max(s));
        const float corr = exp2f(m - m_new);
        const float p = valid ? exp2f(s - m_new) : 0.f;
        l = l * corr + wave_sum(p);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] *= corr;
        const int cnt = (int)((i - j0 + 1) < kWave ? (i - j0 + 1) : kWave);
        for (int jj = 0; jj < cnt; ++jj) {
            const float pj = __shfl(p, jj, kWave);
            const typename E::storage* vr = vh + (j0 + jj) * kvs2;
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = fmaf(pj, load1<E>(vr + lane + r * kWave), acc[r]);
        }
        m = m_new;
    }
    const float inv_l = 1.f / l;
    typename E::storage* orow = o + b * os0 + h * os1 + row * os2;
#pragma unroll
    for (int r = 0; r < R; ++r) store1<E>(orow + lane + r * kWave, acc[r] * inv_l);
}


namespace {

constexpr int kWinWaves = 4;
constexpr int kWinQ = kWinWaves * 32;   // queries per workgroup

template <int D>
struct WinStage {
    static constexpr int KC = kWinQ == 128 ? (mf::kTileK * D / 8) / 256 : 0;  // K chunks / thread
    uint4 k[KC];          // raw bf16 of K rows
    uint4 v[4];           // 4 keys x 8 dims of V (threads < 2D)
};

template <int D>
__device__ __forceinline__ void win_load(WinStage<D>& st, const uint16_t* __restrict__ kh,
                                         const uint16_t* __restrict__ vh, int64_t kvs2, long kt,
                                         long kv_hi, long i0, int w, const float2* __restrict__ table)
{
    // Rows past kv_hi repeat row kv_hi: they lie after every query of the tile, so
    // the tile is masked and their weights are exactly 0.
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < WinStage<D>::KC; ++it) {
        const int c = tid + 256 * it;
        const int kr = c / (D / 8), part = c % (D / 8);
        const long j = kt + kr <= kv_hi ? kt + kr : kv_hi;
        st.k[it] = *reinterpret_cast<const uint4*>(kh + j * kvs2 + part * 8);
    }
    if (tid < 2 * D) {
        // keys 32 grp + 16 hh + 4 g + r (r = 0..3), dims 8 dc .. 8 dc + 7
        const int grp = tid / D, within = tid % D;
        const int hh = within & 1, g = (within >> 1) & 3, dc = within >> 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const long jr = kt + 32 * grp + 16 * hh + 4 * g + r;
            const long j = jr <= kv_hi ? jr : kv_hi;
            st.v[r] = *reinterpret_cast<const uint4*>(vh + j * kvs2 + dc * 8);
        }
    }
}

// Rotate one bf16 pair (x, y) by the angle with cosine c and sine s; pack as fp16.
__device__ __forceinline__ uint32_t rotate_pack(uint32_t xy, float c, float s)
{
    const float x = __uint_as_float(xy << 16), y = __uint_as_float(xy & 0xFFFF0000u);
    return mf::pack_f16x2(x * c - y * s, x * s + y * c);
}

// Rotate the staged keys by R(j - i0) (table read here, L2-resident) and write
// K and V^T to LDS.
template <int D>
__device__ __forceinline__ void win_store(const WinStage<D>& st, uint16_t* ks, uint16_t* vt,
                                          long kt, long kv_hi, long i0, int w,
                                          const float2* __restrict__ table)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < WinStage<D>::KC; ++it) {
        const int c = tid + 256 * it;
        const int kr = c / (D / 8), part = c % (D / 8);
        const long j = kt + kr <= kv_hi ? kt + kr : kv_hi;     // rows past kv_hi repeat it
        const float4* rp = reinterpret_cast<const float4*>(
            table + (j - i0 + w + kTableSlack) * (D / 2) + part * 4);
        const float4 a = rp[0], b = rp[1];
        uint4 o;
        o.x = rotate_pack(st.k[it].x, a.x, a.y);
        o.y = rotate_pack(st.k[it].y, a.z, a.w);
        o.z = rotate_pack(st.k[it].z, b.x, b.y);
        o.w = rotate_pack(st.k[it].w, b.z, b.w);
        mf::lds_store16(ks + mf::ksw_off<D>(kr, part), o);
    }
    if (tid < 2 * D) {
        const int grp = tid / D, within = tid % D;
        const int hh = within & 1, g = (within >> 1) & 3, dc = within >> 3;
        // V^T column slot 8 g + 4 hh + r of the 32-key group holds key 16 hh + 4 g + r
        mf::store_vt_4x8_sw(st.v, vt, dc, 32 * grp + 8 * g + 4 * hh);
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void window_attn_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t kvs0, int64_t kvs1,
    int64_t kvs2, int H, int BH, int nq, int q_pos0, int w, const float2* __restrict__ table,
    float scale_log2, uint16_t* __restrict__ o, int64_t os0, int64_t os1, int64_t os2,
    int n_split, float* __restrict__ ws_acc, float2* __restrict__ ws_ml)
{
    using namespace mf;
    constexpr int KS = D / 32;     // k-steps of the QK^T contraction
    constexpr int DB = D / 16;     // 16-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t ks[kTileK * D];    // swizzled rows
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * kTileK];    // swizzled rows

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int h = (int)(bh % H), b = (int)(bh / H);
    // split `split` of n_split takes a contiguous share of the query tile's key tiles
    const int split = (int)(tb.tile % n_split);
    const long i0 = (long)q_pos0 + (tb.tile / n_split) * kWinQ;
    const long i_end = (long)q_pos0 + nq - 1;                 // last query position
    const long kv_first = i0 - w > 0 ? i0 - w : 0;
    const long kv_hi = i0 + kWinQ - 1 < i_end ? i0 + kWinQ - 1 : i_end;
    const int n_all = (int)((kv_hi - kv_first) / kTileK) + 1;
    const int t_begin = (int)((long)n_all * split / n_split);
    const int n_tiles = (int)((long)n_all * (split + 1) / n_split) - t_begin;
    const long kv_lo = kv_first + (long)t_begin * kTileK;     // first key of this split

    const uint16_t* kh = k + b * kvs0 + h * kvs1;
    const uint16_t* vh = v + b * kvs0 + h * kvs1;

    // this wave's queries: qw0 .. qw0+31 (two groups of 16)
    const long qw0 = i0 + 32 * wv;
    const long qw_last = qw0 + 31 < i_end ? qw0 + 31 : i_end;
    const bool wave_active = qw0 <= i_end;

    // rotated queries as B operands, kept for the whole key range
    f16x8 qf[2][KS];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const long i = qw0 + 16 * qg + n;
        const bool ok = i <= i_end;
        const uint16_t* qrow = q + b * qs0 + h * qs1 + (ok ? i - q_pos0 : 0) * qs2;
        const float2* rot = table + (ok ? i - i0 + w + kTableSlack : w + kTableSlack) * (D / 2);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            uint4 raw = ok ? *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * g)
                           : make_uint4(0, 0, 0, 0);
            const float4* rp = reinterpret_cast<const float4*>(rot + 16 * t + 4 * g);
            const float4 a = rp[0], c = rp[1];
            uint4 u;
            u.x = rotate_pack(raw.x, a.x, a.y);
            u.y = rotate_pack(raw.y, a.z, a.w);
            u.z = rotate_pack(raw.z, c.x, c.y);
            u.w = rotate_pack(raw.w, c.z, c.w);
            qf[qg][t] = as_f16x8(u);
        }
    }

    f32x4 acc[DB][2], accl[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    accl[0] = accl[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};

    WinStage<D> stage;
    if (n_tiles > 0) {                                        // block-uniform
        win_load<D>(stage, kh, vh, kvs2, kv_lo, kv_hi, i0, w, table);
        win_store<D>(stage, ks, vt, kv_lo, kv_hi, i0, w, table);
    }
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
        const long kt = kv_lo + (long)tile * kTileK;
        if (tile + 1 < n_tiles)
            win_load<D>(stage, kh, vh, kvs2, kt + kTileK, kv_hi, i0, w, table);

        // does any query of this wave see a key of this tile?
        const bool work = wave_active && kt <= qw_last && kt + kTileK - 1 >= qw0 - w;
        if (work) {
            // every key of the tile inside every query's window: no masking needed
            const bool full = kt >= qw_last - w && kt + kTileK - 1 <= qw0;
            // i - j for query 16 qg + n and key 16 kb + 4 g + r, in 32 bits (|i - j| < 2^31)
            const int d0 = (int)(qw0 - kt) + n - 4 * g;
            auto keep = [&](int kb, int qg, int r) {
                const int d = d0 + 16 * (qg - kb) - r;
                return d >= 0 && d <= w;
            };
            attn_tile<D>(ks, vt, qf, acc, accl, m_run, scale_log2, !full, keep);
        }
        __syncthreads();
        if (tile + 1 < n_tiles) {
            win_store<D>(stage, ks, vt, kt + kTileK, kv_hi, i0, w, table);
            __syncthreads();
        }
    }

    if (n_split > 1) {                  // partial state (m, l, unnormalised O) of this split
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const long i = qw0 + 16 * qg + n;
            if (i > i_end) continue;
            const long slot = (bh * nq + (i - q_pos0)) * n_split + split;
            if (g == 0) ws_ml[slot] = make_float2(m_run[qg], accl[qg][0]);
            float* dst = ws_acc + slot * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *reinterpret_cast<float4*>(dst + 16 * db + 4 * g) =
                    make_float4(acc[db][qg][0], acc[db][qg][1], acc[db][qg][2], acc[db][qg][3]);
        }
        return;
    }
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const long i = qw0 + 16 * qg + n;
        const float l = accl[qg][0];    // every row of the ones product is the full sum
        if (i > i_end) continue;
        const float inv = 1.f / l;
        uint16_t* orow = o + b * os0 + h * os1 + (i - q_pos0) * os2;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            uint2 u;
            u.x = cvt_pk_bf16(acc[db][qg][0] * inv, acc[db][qg][1] * inv);
            u.y = cvt_pk_bf16(acc[db][qg][2] * inv, acc[db][qg][3] * inv);
            *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g) = u;
        }
    }
}

hipError_t launch_rope_table(const Shape& sh, double rope_base, void* table, hipStream_t st)
{
    const int rows = sh.w + 2 * kTableSlack, half = sh.d / 2;
    const long n_tab = (long)rows * half;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n_tab + 255) / 256)), dim3(256), 0, st,
                       (float2*)table, rows, half, sh.w, log(rope_base));
    return hipGetLastError();
}

// Splits of each query tile's key range: enough workgroups to give every CU two,
// at most one per key tile and 16 in all (bf16 storage only).
int window_splits(const Shape& sh)
{
    if (!sh.bf16 || sh.nq == 0) return 1;
    const long base = (sh.nq + kWinQ - 1) / kWinQ * (long)sh.B * sh.H;
    if (base >= 512) return 1;
    const long tiles = (sh.w + kWinQ - 1) / mf::kTileK + 1;       // key tiles of a query tile, at most
    long want = (512 + base - 1) / base;
    want = want < tiles ? want : tiles;
    return (int)(want < 16 ? want : 16);
}

size_t window_ws_bytes(const Shape& sh)
{
    const int S = window_splits(sh);
    if (S <= 1) return 0;
    const size_t rows = (size_t)sh.B * sh.H * sh.nq * S;
    return rows * ((size_t)sh.d * sizeof(float) + sizeof(float2));
}

size_t window_workspace_bytes(const Shape& sh)
{
    return ((rope_table_bytes(sh) + 255) & ~(size_t)255) + window_ws_bytes(sh);
}

hipError_t launch_window(const Shape& sh, const void* q, const void* k, const void* v,
                         double rope_base, void* table, void* o_sr, hipStream_t st,
                         bool table_ready, size_t ws_bytes)
{
    if (sh.nq == 0) return hipSuccess;
    if (!table_ready) {
        const hipError_t err = launch_rope_table(sh, rope_base, table, st);
        if (err != hipSuccess) return err;
    }
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)sh.d));
    if (sh.bf16) {
        // split the key range when the workspace holds the partial states
        const int S = ws_bytes >= window_workspace_bytes(sh) ? window_splits(sh) : 1;
        char* wsb = static_cast<char*>(table) + ((rope_table_bytes(sh) + 255) & ~(size_t)255);
        const long rows_all = (long)sh.B * sh.H * sh.nq;
        float* ws_acc = S > 1 ? reinterpret_cast<float*>(wsb) : nullptr;
        float2* ws_ml = S > 1 ? reinterpret_cast<float2*>(ws_acc + rows_all * S * sh.d) : nullptr;
        const long n_tiles = (sh.nq + kWinQ - 1) / kWinQ;
        dim3 grid((unsigned)(n_tiles * S * sh.B * sh.H)), block(256);
#define FS_WINDOW_MFMA(D)                                                                        \
        hipLaunchKernelGGL((window_attn_mfma_kernel<D>), grid, block, 0, st, (const uint16_t*)q,  \
                           sh.qs[0], sh.qs[1], sh.qs[2], (const uint16_t*)k, (const uint16_t*)v,  \
                           sh.kvs[0], sh.kvs[1], sh.kvs[2], sh.H, sh.B * sh.H, sh.nq, sh.q_pos0,  \
                           sh.w,                                                                  \
                           (const float2*)table, scale_log2, (uint16_t*)o_sr, sh.os[0], sh.os[1], \
                           sh.os[2], S, ws_acc, ws_ml)
        if (sh.d == 64) FS_WINDOW_MFMA(64); else FS_WINDOW_MFMA(128);
#undef FS_WINDOW_MFMA
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess || S <= 1) return err;
        return launch_split_merge(sh, S, ws_acc, ws_ml, false, 0.f, o_sr, st);
    }
    dim3 grid((unsigned)((sh.nq + 3) / 4), (unsigned)(sh.B * sh.H)), block(256);
#define FS_WINDOW(E, D)                                                                          \
    hipLaunchKernelGGL((window_attn_rowwise_kernel<E, D>), grid, block, 0, st,                   \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2],              \
                       (const typename E::storage*)k, (const typename E::storage*)v, sh.kvs[0],  \
                       sh.kvs[1], sh.kvs[2], sh.H, sh.nq, sh.q_pos0, sh.w,                       \
                       (const float2*)table, scale_log2, (typename E::storage*)o_sr, sh.os[0],   \
                       sh.os[1], sh.os[2])
    if (sh.d == 64) FS_WINDOW(F32, 64); else FS_WINDOW(F32, 128);
#undef FS_WINDOW
    return hipGetLastError();
}

}  // namespace fs
