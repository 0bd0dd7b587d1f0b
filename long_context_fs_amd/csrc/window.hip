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
// the same MFMA rate).  fp16 stops at 65504, so each wave's queries and each key
// tile are scaled by a power of two 2^-e before packing, e the smallest shift
// that keeps every rotated element below 2^15 (taken from the bf16 exponents;
// blocks of tiny values are scaled up instead; 0 for ordinary inputs), and the
// logits by 2^(e_q + e_k) after the product: exact, and any finite bf16 input
// gives a finite output.
// Per tile a wave computes S^T = K Q^T (16x16x32 fp16 MFMA, fp32 accumulate),
// masks to max(0, i-w) <= j <= i, runs the online
// softmax in fp32 (exp2 with log2(e)/sqrt(d) folded into the scale), and
// accumulates O^T += V^T P^T with P rounded to bf16.  The next tile's global
// loads are issued before the current tile's MFMAs (register double buffer).
// When the query tiles alone would leave the chip idle (decode), a tile's key
// range is split over workgroups whose partial (max, sum, O) states the
// readout's merge kernel combines.
// f32 storage: the same tiles on the fp32 matrix product (below).
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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running maximum of the bf16 magnitudes (sign cleared; they order like the
// values) of the 8 bf16 values in u, two lanes of 16 bits.
__device__ __forceinline__ u16x2 max_bf16_mag(u16x2 m, const uint4& u)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        m = __builtin_elementwise_max(
            m, __builtin_bit_cast(u16x2, mf::word_of(u, i) & 0x7FFF7FFFu));
    return m;
}

// Biased exponent field of the larger of the two magnitudes.
__device__ __forceinline__ uint32_t mag_exp(u16x2 m) { return (uint32_t)max(m.x, m.y) >> 7; }

// Largest biased exponent field of the 8 bf16 values in u.
__device__ __forceinline__ uint32_t max_bf16_exp(const uint4& u)
{
    return mag_exp(max_bf16_mag(u16x2{0, 0}, u));
}

// Shift e of a block whose largest bf16 exponent field is E: a rotated pair has
// norm <= sqrt(2) * 2^(E - 126) < 2^(E - 125), and 2^(E - 125 - e) <= 2^15 keeps
// it inside fp16.  A block of tiny values (largest below 2^-15, where fp16 is
// subnormal) is scaled up to a largest value near 1.  In between, e = 0.
__device__ __forceinline__ int fp16_shift(uint32_t E)
{
    if (E > 140u) return (int)E - 140;
    if (E < 112u) return E > 27u ? (int)E - 127 : -100;   // (all zero: any shift)
    return 0;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, m, kWave));
    return x;
}

// Rotate the staged keys by R(j - i0) (table read here, L2-resident) and write
// K and V^T to LDS.
template <int D>
__device__ __forceinline__ void win_store(const WinStage<D>& st, uint16_t* ks, uint16_t* vt,
                                          long kt, long kv_hi, long i0, int w,
                                          const float2* __restrict__ table, int e_k)
{
    const int tid = threadIdx.x;
    const float sc = ldexpf(1.f, -e_k);                         // exact power of two
#pragma unroll
    for (int it = 0; it < WinStage<D>::KC; ++it) {
        const int c = tid + 256 * it;
        const int kr = c / (D / 8), part = c % (D / 8);
        const long j = kt + kr <= kv_hi ? kt + kr : kv_hi;     // rows past kv_hi repeat it
        const float4* rp = reinterpret_cast<const float4*>(
            table + (j - i0 + w + kTableSlack) * (D / 2) + part * 4);
        float4 a = rp[0], b = rp[1];
        if (e_k != 0) {                                         // block-uniform
            a.x *= sc; a.y *= sc; a.z *= sc; a.w *= sc;
            b.x *= sc; b.y *= sc; b.z *= sc; b.w *= sc;
        }
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

// Each wave's largest exponent of the staged raw keys, into red[wave]; the
// exact maximum is only formed when some value is outside the shift-free range
// (a ballot), otherwise a value inside it stands for the wave.
template <int D>
__device__ __forceinline__ void win_key_exp(const WinStage<D>& st, uint32_t* red)
{
    u16x2 mm = {0, 0};
#pragma unroll
    for (int it = 0; it < WinStage<D>::KC; ++it) mm = max_bf16_mag(mm, st.k[it]);
    uint32_t m = mag_exp(mm);
    const bool big = __ballot(m > 140u) != 0, tiny = __ballot(m >= 112u) == 0;
    m = (big || tiny) ? wave_max_u32(m) : 127u;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
}

__device__ __forceinline__ int win_block_shift(const uint32_t* red)
{
    return fp16_shift(max(max(red[0], red[1]), max(red[2], red[3])));
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
    __shared__ uint32_t kexp[kWinWaves];                                 // per-wave key exponents

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

    // rotated queries as B operands, kept for the whole key range, scaled by the
    // wave's 2^-e_q
    f16x8 qf[2][KS];
    uint4 qraw[2][KS];
    uint32_t qe = 0;
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const long i = qw0 + 16 * qg + n;
        const bool ok = i <= i_end;
        const uint16_t* qrow = q + b * qs0 + h * qs1 + (ok ? i - q_pos0 : 0) * qs2;
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            qraw[qg][t] = ok ? *reinterpret_cast<const uint4*>(qrow + 32 * t + 8 * g)
                             : make_uint4(0, 0, 0, 0);
            qe = max(qe, max_bf16_exp(qraw[qg][t]));
        }
    }
    const int e_q = fp16_shift(wave_max_u32(qe));
    const float q_sc = ldexpf(1.f, -e_q);
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const long i = qw0 + 16 * qg + n;
        const bool ok = i <= i_end;
        const float2* rot = table + (ok ? i - i0 + w + kTableSlack : w + kTableSlack) * (D / 2);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const uint4 raw = qraw[qg][t];
            const float4* rp = reinterpret_cast<const float4*>(rot + 16 * t + 4 * g);
            float4 a = rp[0], c = rp[1];
            if (e_q != 0) {                                     // wave-uniform
                a.x *= q_sc; a.y *= q_sc; a.z *= q_sc; a.w *= q_sc;
                c.x *= q_sc; c.y *= q_sc; c.z *= q_sc; c.w *= q_sc;
            }
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
    int e_k = 0;                                              // the staged tile's key shift
    if (n_tiles > 0) {                                        // block-uniform
        win_load<D>(stage, kh, vh, kvs2, kv_lo, kv_hi, i0, w, table);
        win_key_exp<D>(stage, kexp);
        __syncthreads();
        e_k = win_block_shift(kexp);
        win_store<D>(stage, ks, vt, kv_lo, kv_hi, i0, w, table, e_k);
    }
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
        const long kt = kv_lo + (long)tile * kTileK;
        if (tile + 1 < n_tiles)
            win_load<D>(stage, kh, vh, kvs2, kt + kTileK, kv_hi, i0, w, table);
        // logits of this tile: the scaled product times 2^(e_q + e_k)
        const float scale_t = (e_q + e_k) == 0 ? scale_log2 : ldexpf(scale_log2, e_q + e_k);

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
            attn_tile<D>(ks, vt, qf, acc, accl, m_run, scale_t, !full, keep);
        }
        if (tile + 1 < n_tiles) win_key_exp<D>(stage, kexp);     // the next tile's keys
        __syncthreads();
        if (tile + 1 < n_tiles) {
            e_k = win_block_shift(kexp);
            win_store<D>(stage, ks, vt, kt + kTileK, kv_hi, i0, w, table, e_k);
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

// ---- fp32 storage on the matrix core ------------------------------------------
//
// The same workgroup shape and key tiles as the bf16 kernel, on the fp32
// product v_mfma_f32_16x16x4f32 (exact fp32 products, fp32 sums), so fp32
// inputs keep fp32 accuracy and need no operand range care.  The QK^T
// contraction over d runs as D/4 steps in which lane group g supplies dimension
// g*D/4 + t: a lane reads its key row's D/4 consecutive floats (16-byte LDS
// reads) and holds its query's D/4 consecutive rotated floats.  For PV, step j
// of a 16-key block contracts keys 4g + j, which is register j of the lane's S^T
// fragment, so P needs no movement; V is read from a row-major LDS tile.  Rows
// are padded by 16 bytes against LDS bank conflicts.  The softmax sum is kept
// per lane and reduced over the four lanes of a query at the end.

namespace {

constexpr int kF32Pad = 4;                 // floats of row padding

template <int D>
struct WinStageF32 {
    static constexpr int KC = (mf::kTileK * D / 4) / 256;   // 16-byte chunks of K per thread
    float4 k[KC];
    float4 v[KC];
};

template <int D>
__device__ __forceinline__ void winf_load(WinStageF32<D>& st, const float* __restrict__ kh,
                                          const float* __restrict__ vh, int64_t kvs2, long kt,
                                          long kv_hi)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < WinStageF32<D>::KC; ++it) {
        const int c = tid + 256 * it;
        const int kr = c / (D / 4), part = c % (D / 4);
        const long j = kt + kr <= kv_hi ? kt + kr : kv_hi;   // rows past kv_hi repeat it
        st.k[it] = *reinterpret_cast<const float4*>(kh + j * kvs2 + part * 4);
        st.v[it] = *reinterpret_cast<const float4*>(vh + j * kvs2 + part * 4);
    }
}

// K rotated by R(j - i0) and V, row-major with padded rows, into LDS.
template <int D>
__device__ __forceinline__ void winf_store(const WinStageF32<D>& st, float* ks, float* vs, long kt,
                                           long kv_hi, long i0, int w,
                                           const float2* __restrict__ table)
{
    constexpr int P = D + kF32Pad;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < WinStageF32<D>::KC; ++it) {
        const int c = tid + 256 * it;
        const int kr = c / (D / 4), part = c % (D / 4);
        const long j = kt + kr <= kv_hi ? kt + kr : kv_hi;
        const float4 cs = *reinterpret_cast<const float4*>(
            table + (j - i0 + w + kTableSlack) * (D / 2) + part * 2);
        const float4 x = st.k[it];
        float4 r;
        r.x = x.x * cs.x - x.y * cs.y;
        r.y = x.x * cs.y + x.y * cs.x;
        r.z = x.z * cs.z - x.w * cs.w;
        r.w = x.z * cs.w + x.w * cs.z;
        *reinterpret_cast<float4*>(ks + kr * P + part * 4) = r;
        *reinterpret_cast<float4*>(vs + kr * P + part * 4) = st.v[it];
    }
}

}  // namespace

// d128 holds 2 x 32 rotated query floats, 2 x 32 accumulators and a 16 KiB-per-tile
// register stage per lane, which only fit at one wave per SIMD.
template <int D>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void window_attn_f32_kernel(
    const float* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ k, const float* __restrict__ v, int64_t kvs0, int64_t kvs1,
    int64_t kvs2, int H, int BH, int nq, int q_pos0, int w, const float2* __restrict__ table,
    float scale_log2, float* __restrict__ o, int64_t os0, int64_t os1, int64_t os2,
    int n_split, float* __restrict__ ws_acc, float2* __restrict__ ws_ml)
{
    using namespace mf;
    constexpr int T = D / 4;       // contraction steps over d; floats per lane and row
    constexpr int DB = D / 16;     // 16-row blocks of O^T
    constexpr int P = D + kF32Pad;
    __shared__ __attribute__((aligned(16))) float ks[kTileK * P];
    __shared__ __attribute__((aligned(16))) float vs[kTileK * P];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const TileOfBlock tb = xcd_tile(BH);
    const long bh = tb.bh;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int split = (int)(tb.tile % n_split);
    const long i0 = (long)q_pos0 + (tb.tile / n_split) * kWinQ;
    const long i_end = (long)q_pos0 + nq - 1;
    const long kv_first = i0 - w > 0 ? i0 - w : 0;
    const long kv_hi = i0 + kWinQ - 1 < i_end ? i0 + kWinQ - 1 : i_end;
    const int n_all = (int)((kv_hi - kv_first) / kTileK) + 1;
    const int t_begin = (int)((long)n_all * split / n_split);
    const int n_tiles = (int)((long)n_all * (split + 1) / n_split) - t_begin;
    const long kv_lo = kv_first + (long)t_begin * kTileK;

    const float* kh = k + b * kvs0 + h * kvs1;
    const float* vh = v + b * kvs0 + h * kvs1;
    const long qw0 = i0 + 32 * wv;
    const long qw_last = qw0 + 31 < i_end ? qw0 + 31 : i_end;
    const bool wave_active = qw0 <= i_end;

    // lane (n, g): dims g*T .. g*T+T-1 of query 16 qg + n, rotated by R(i - i0)
    float qf[2][T];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        const long i = qw0 + 16 * qg + n;
        const bool ok = i <= i_end;
        const float* qrow = q + b * qs0 + h * qs1 + (ok ? i - q_pos0 : 0) * qs2 + g * T;
        const float2* rot = table + (ok ? i - i0 + w + kTableSlack : w + kTableSlack) * (D / 2) +
                            g * (T / 2);
#pragma unroll
        for (int c = 0; c < T / 4; ++c) {
            const float4 x = ok ? *reinterpret_cast<const float4*>(qrow + 4 * c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 cs = *reinterpret_cast<const float4*>(rot + 2 * c);
            qf[qg][4 * c + 0] = x.x * cs.x - x.y * cs.y;
            qf[qg][4 * c + 1] = x.x * cs.y + x.y * cs.x;
            qf[qg][4 * c + 2] = x.z * cs.z - x.w * cs.w;
            qf[qg][4 * c + 3] = x.z * cs.w + x.w * cs.z;
        }
    }

    f32x4 acc[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float l_part[2] = {0.f, 0.f};              // this lane's share of the softmax sums
    float m_run[2] = {-INFINITY, -INFINITY};

    WinStageF32<D> stage;
    if (n_tiles > 0) {
        winf_load<D>(stage, kh, vh, kvs2, kv_lo, kv_hi);
        winf_store<D>(stage, ks, vs, kv_lo, kv_hi, i0, w, table);
    }
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
        const long kt = kv_lo + (long)tile * kTileK;
        if (tile + 1 < n_tiles) winf_load<D>(stage, kh, vh, kvs2, kt + kTileK, kv_hi);
        const bool work = wave_active && kt <= qw_last && kt + kTileK - 1 >= qw0 - w;
        if (work) {
            const bool full = kt >= qw_last - w && kt + kTileK - 1 <= qw0;
            const int d0 = (int)(qw0 - kt) + n - 4 * g;   // i - j for key 16 kb + 4 g + r
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
                if (!full) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int dd = d0 + 16 * (qg - kb) - r;
                            if (!(dd >= 0 && dd <= w)) s[kb][qg][r] = -INFINITY;
                        }
                }
                float tmax = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        tmax = __builtin_elementwise_maximum(tmax, s[kb][qg][r]);
                tmax = xrow_max(tmax) * scale_log2;
                const bool raise = tmax > m_run[qg] + kLazy;
                const float m_new = raise ? tmax : m_run[qg];
                corr[qg] = raise ? __builtin_amdgcn_exp2f(m_run[qg] - m_new) : 1.f;
                any_rescale |= raise;
                m_run[qg] = m_new;
                const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        s[kb][qg][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qg][r], scale_log2, neg_m));
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
            // O^T += V^T P^T: step (kb, j) contracts keys 16 kb + 4 g + j
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
        if (tile + 1 < n_tiles) {
            winf_store<D>(stage, ks, vs, kt + kTileK, kv_hi, i0, w, table);
            __syncthreads();
        }
    }

    float l[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) l[qg] = xrow_sum(l_part[qg]);
    if (n_split > 1) {
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
            const long i = qw0 + 16 * qg + n;
            if (i > i_end) continue;
            const long slot = (bh * nq + (i - q_pos0)) * n_split + split;
            if (g == 0) ws_ml[slot] = make_float2(m_run[qg], l[qg]);
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
        if (i > i_end) continue;
        const float inv = 1.f / l[qg];
        float* orow = o + b * os0 + h * os1 + (i - q_pos0) * os2;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<float4*>(orow + 16 * db + 4 * g) =
                make_float4(acc[db][qg][0] * inv, acc[db][qg][1] * inv, acc[db][qg][2] * inv,
                            acc[db][qg][3] * inv);
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
// at most one per key tile and 16 in all.
int window_splits(const Shape& sh)
{
    if (sh.nq == 0) return 1;
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
    // split the key range when the workspace holds the partial states
    const int S = ws_bytes >= window_workspace_bytes(sh) ? window_splits(sh) : 1;
    char* wsb = static_cast<char*>(table) + ((rope_table_bytes(sh) + 255) & ~(size_t)255);
    const long rows_all = (long)sh.B * sh.H * sh.nq;
    float* ws_acc = S > 1 ? reinterpret_cast<float*>(wsb) : nullptr;
    float2* ws_ml = S > 1 ? reinterpret_cast<float2*>(ws_acc + rows_all * S * sh.d) : nullptr;
    const long n_tiles = (sh.nq + kWinQ - 1) / kWinQ;
    dim3 grid((unsigned)(n_tiles * S * sh.B * sh.H)), block(256);
    if (!sh.bf16) {
        note_path("window: fp32 MFMA tiles of 128 queries, %d split(s)", S);
#define FS_WINDOW_F32(D)                                                                         \
        hipLaunchKernelGGL((window_attn_f32_kernel<D>), grid, block, 0, st, (const float*)q,      \
                           sh.qs[0], sh.qs[1], sh.qs[2], (const float*)k, (const float*)v,        \
                           sh.kvs[0], sh.kvs[1], sh.kvs[2], sh.H, sh.B * sh.H, sh.nq, sh.q_pos0,  \
                           sh.w, (const float2*)table, scale_log2, (float*)o_sr, sh.os[0],        \
                           sh.os[1], sh.os[2], S, ws_acc, ws_ml)
        if (sh.d == 64) FS_WINDOW_F32(64); else FS_WINDOW_F32(128);
#undef FS_WINDOW_F32
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess || S <= 1) return err;
        return launch_split_merge(sh, S, ws_acc, ws_ml, false, 0.f, o_sr, st);
    }
    {
        note_path("window: MFMA tiles of 128 queries, %d split(s)", S);
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
}

}  // namespace fs
