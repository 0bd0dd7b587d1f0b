// mfma_tile.hpp -- bf16 MFMA building blocks of the flash-style attention tiles.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16, n = l % 16):
//   A (16 x 32): lane holds row n, k = 8g .. 8g+7        (8 bf16, 16 bytes)
//   B (32 x 16): lane holds column n, k = 8g .. 8g+7
//   C (16 x 16): lane holds column n, rows 4g .. 4g+3    (4 floats)
//
// The tiles compute S^T = K Q^T (keys as rows, queries as columns), so a lane's
// C registers are 4 keys of ONE query: the softmax statistics of a query live
// in the 4 lanes n, n+16, n+32, n+48.  Two 16-key S^T blocks give a lane the
// keys {4g..4g+3} and {16+4g..16+4g+3} of a 32-key group, exactly the 8 values
// the B operand of O^T += V^T P^T needs, if k-slot 8g+j stands for key
//   pi(8g+j) = 4g+j (j < 4),  16+4g+(j-4) (j >= 4).
// V^T is therefore stored in LDS with its columns in that order: column
// 8g+4h+r of a 32-key group holds key 16h+4g+r.
#pragma once

#include "fs_device.hpp"

namespace fs {
namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileK = 64;               // keys per tile

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f16x8 as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8, u); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
// 32x32x16 bf16 product: lane l holds A row l % 32 and B column l % 32 with
// k = 8 (l / 32) .. + 7; C register e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4
// of column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp32 16x16x4 product (exact fp32 products, fp32 sums): lane l holds A row l % 16
// and B column l % 16 at k = l / 16; C register r of lane l is row 4 (l / 16) + r
// of column l % 16.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even float -> fp16 bits, two values per dword (low first).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    const uint32_t a = __builtin_bit_cast(uint16_t, (_Float16)lo);
    const uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)hi);
    return a | (b << 16);
}

__device__ __forceinline__ uint4 lds_load16(const uint16_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void lds_store16(uint16_t* p, uint4 v)
{
    *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int i)
{
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// ---- XOR-swizzled tiles (unpadded) ------------------------------------------
// gfx950 LDS has 64 banks (a 256-byte period) and serves a 16-byte-per-lane
// access 16 lanes at a time, in the interleaved groups {0-3, 12-15, 20-23,
// 24-27}, {4-11, 16-19, 28-31} (and the same for lanes 32-63), as measured with
// the bank-conflict counters.  An MFMA fragment read (lane (n, g) reads chunk
// 4t + g of row n) therefore has no conflict exactly when the 16-byte bank slot
// it hits depends on n alone.  The swizzled tiles store chunk c of row r at
// chunk position c ^ sw(r), with sw(r) = the index of r's 256-byte period
// modulo the chunks per row, which gives every row a distinct slot for a fixed
// c up to the bits that g flips -- and keeps the row-wise stores conflict-free.
template <int ROW>   // bf16 elements per row: 64 or 128
__device__ __forceinline__ int sw_off(int row, int chunk)
{
    constexpr int kChunks = ROW / 8, kRowsPer256 = 128 / ROW;
    return row * ROW + ((chunk ^ ((row / kRowsPer256) & (kChunks - 1))) << 3);
}

// K tile: rows of D bf16.
template <int D>
__device__ __forceinline__ int ksw_off(int row, int chunk) { return sw_off<D>(row, chunk); }

// V^T tile: D rows of 64 key-permuted bf16.
__device__ __forceinline__ int vtsw_off(int row, int chunk) { return sw_off<kTileK>(row, chunk); }

// store_vt_4x8 for the swizzled V^T tile: dims 8 dc .. 8 dc + 7, key columns
// col .. col + 3 (col a multiple of 4).
__device__ __forceinline__ void store_vt_4x8_sw(const uint4 in[4], uint16_t* vt, int dc, int col)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t a0 = word_of(in[0], e >> 1), a1 = word_of(in[1], e >> 1);
        const uint32_t a2 = word_of(in[2], e >> 1), a3 = word_of(in[3], e >> 1);
        // one byte permute per dword: the low (even e) or high (odd e) halves of
        // two rows, first row low (v_perm_b32 selectors 0-3 pick src1's bytes)
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint2 w;
        w.x = __builtin_amdgcn_perm(a1, a0, sel);
        w.y = __builtin_amdgcn_perm(a3, a2, sel);
        *reinterpret_cast<uint2*>(vt + vtsw_off(dc * 8 + e, col >> 3) + (col & 4)) = w;
    }
}


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even, v_cvt_pk_bf16_f32), low first.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Pack 8 probabilities (keys pi(8g+0..7)) into the B operand of O^T += V^T P^T.
__device__ __forceinline__ bf16x8 pack_p(const f32x4& lo, const f32x4& hi)
{
    uint4 u;
    u.x = cvt_pk_bf16(lo[0], lo[1]);
    u.y = cvt_pk_bf16(lo[2], lo[3]);
    u.z = cvt_pk_bf16(hi[0], hi[1]);
    u.w = cvt_pk_bf16(hi[2], hi[3]);
    return as_bf16x8(u);
}

// Max / sum over the lanes l, l^16, l^32, l^48 (one query's four lane groups),
// with the gfx950 row-swap permutes (VALU, no LDS round trip).
// (IEEE maximum, which needs no canonicalising of the permuted operands)
__device__ __forceinline__ float xrow_max(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xrow_sum(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Rescale threshold of the online softmax (log2 units): the running reference
// max is only raised when a tile's max exceeds it by more than this, so the
// accumulators are rarely rescaled; probabilities stay <= 2^kLazy.
constexpr float kLazy = 8.f;

// One 64-key tile of flash attention for a wave's 32 queries (two groups of 16).
//   ks : swizzled K tile in LDS, 64 rows of D (ksw_off), element type of Frag
//   vt : swizzled V^T tile in LDS, D rows of 64 key-permuted bf16 (vtsw_off)
//   qf : the queries as B operands, qf[qg][t] = dims 32t + 8g .. + 7 of query 16 qg + n
//   masked          : whether some key of the tile may be hidden from some query
//                     (wave-uniform; when false, keep is not evaluated)
//   keep(kb, qg, r) : whether key 16 kb + 4 g + r is visible to query 16 qg + n
// Updates the reference max m_ref (log2 domain, raised lazily), the O^T
// accumulators and accl, the softmax denominator accumulated on the matrix core
// as P^T times a row of ones (every row of accl[qg] holds the running sum).
template <int D, class Frag, class Keep>
__device__ __forceinline__ void attn_tile(const uint16_t* ks, const uint16_t* vt,
                                          const Frag (&qf)[2][D / 32], f32x4 (&acc)[D / 16][2],
                                          f32x4 (&accl)[2], float (&m_ref)[2], float scale_log2,
                                          bool masked, Keep keep)
{
    constexpr int KS = D / 32, DB = D / 16;
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const Frag a = __builtin_bit_cast(Frag, lds_load16(ks + ksw_off<D>(16 * kb + n, 4 * t + g)));
            s[kb][0] = mfma(a, qf[0][t], s[kb][0]);
            s[kb][1] = mfma(a, qf[1][t], s[kb][1]);
        }
    }
    bf16x8 pf[2][2];
    float corr[2];
    bool any_rescale = false;
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
        if (masked) {   // one code path for both kinds of tile: no register copies at the join
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!keep(kb, qg, r)) s[kb][qg][r] = -INFINITY;
        }
        // max of the raw scores (scale_log2 > 0 commutes with max)
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)   // IEEE maximum: no NaN quieting of MFMA results
                tmax = __builtin_elementwise_maximum(tmax, s[kb][qg][r]);
        tmax = xrow_max(tmax) * scale_log2;
        // raise the reference only when the tile max exceeds it by > kLazy
        const bool raise = tmax > m_ref[qg] + kLazy;
        const float m_new = raise ? tmax : m_ref[qg];
        corr[qg] = raise ? __builtin_amdgcn_exp2f(m_ref[qg] - m_new) : 1.f;   // 0 at the start
        any_rescale |= raise;
        m_ref[qg] = m_new;
        const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                // v_exp_f32: results below 2^-126 flush to 0, harmless for weights
                s[kb][qg][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qg][r], scale_log2, neg_m));
        }
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
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
            const bf16x8 a = as_bf16x8(lds_load16(vt + vtsw_off(16 * db + n, 4 * a2 + g)));
            acc[db][0] = mfma(a, pf[a2][0], acc[db][0]);
            acc[db][1] = mfma(a, pf[a2][1], acc[db][1]);
        }
    }
    // after the PV products, so that the no-rescale path needs no register copies
    const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
        accl[0] = mfma(ones, pf[a2][0], accl[0]);
        accl[1] = mfma(ones, pf[a2][1], accl[1]);
    }
}

}  // namespace mf
}  // namespace fs
