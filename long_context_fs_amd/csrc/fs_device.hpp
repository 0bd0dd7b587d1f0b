// fs_device.hpp -- device helpers shared by the FS-L kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fs {

constexpr int kWave = 64;

// ---- element types ---------------------------------------------------------
// bf16 is carried as its 16-bit pattern; f32 as float.
struct Bf16 {
    using storage = uint16_t;
    static constexpr int kPer16B = 8;
};
struct F32 {
    using storage = float;
    static constexpr int kPer16B = 4;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Load 16 bytes = E::kPer16B elements and widen to float.
template <class E>
__device__ __forceinline__ void load16(const typename E::storage* p, float* out);

template <>
__device__ __forceinline__ void load16<Bf16>(const uint16_t* p, float* out) {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(a[i] << 16);
        out[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load16<F32>(const float* p, float* out) {
    float4 w = *reinterpret_cast<const float4*>(p);
    out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
}

// Store E::kPer16B floats as 16 bytes of E.
template <class E>
__device__ __forceinline__ void store16(typename E::storage* p, const float* in);

template <>
__device__ __forceinline__ void store16<Bf16>(uint16_t* p, const float* in) {
    uint4 w;
    w.x = pack_bf16x2(in[0], in[1]);
    w.y = pack_bf16x2(in[2], in[3]);
    w.z = pack_bf16x2(in[4], in[5]);
    w.w = pack_bf16x2(in[6], in[7]);
    *reinterpret_cast<uint4*>(p) = w;
}

template <>
__device__ __forceinline__ void store16<F32>(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
}

template <class E>
__device__ __forceinline__ float load1(const typename E::storage* p);
template <>
__device__ __forceinline__ float load1<Bf16>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load1<F32>(const float* p) { return *p; }

template <class E>
__device__ __forceinline__ void store1(typename E::storage* p, float x);
template <>
__device__ __forceinline__ void store1<Bf16>(uint16_t* p, float x) { *p = (uint16_t)f32_to_bf16(x); }
template <>
__device__ __forceinline__ void store1<F32>(float* p, float x) { *p = x; }

// ---- wave reductions (64 lanes) ---------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
    return x;
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum / max over the 16 lanes of a DPP row (lanes 16r .. 16r+15), result in
// every lane of the row: swap neighbours, swap pairs, mirror halves, mirror row.
__device__ __forceinline__ int row16_sum(int x)
{
    x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);   // row_half_mirror
    x += __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);   // row_mirror
    return x;
}

// Sum over the 4 consecutive lanes of a quad, result in every lane of the quad.
__device__ __forceinline__ int quad_sum(int x)
{
    x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    return x;
}

// Exclusive prefix sum over the lanes of a quad (lane 4q+j gets the sum of lanes 4q..4q+j-1).
__device__ __forceinline__ int quad_excl_prefix(int x)
{
    const int j = __lane_id() & 3;
    const int x0 = __builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, false);   // lane 4q
    const int x1 = __builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, false);   // lane 4q+1
    const int x2 = __builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, false);   // lane 4q+2
    return (j > 0 ? x0 : 0) + (j > 1 ? x1 : 0) + (j > 2 ? x2 : 0);
}

__device__ __forceinline__ uint32_t row16_min_u32(uint32_t x)
{
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));
    return x;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Total order on finite floats as unsigned keys (larger float -> larger key).
// Key 0 is below every finite float and marks "no candidate".
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup -> (head, query tile) mapping for 1-D grids of n_tiles * BH blocks.
// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8),
// each with its own L2.  Making the head the fastest-varying index keeps every
// block of one head on the same XCD, so that head's K/V (or kbar) working set
// is cached in one L2 instead of all eight; query tiles advance together.
struct TileOfBlock {
    long bh;
    long tile;
};
__device__ __forceinline__ TileOfBlock xcd_tile(long BH)
{
    const long bid = blockIdx.x;
    return TileOfBlock{bid % BH, bid / BH};
}

// Candidate count of the query at absolute position i: complete cells whose
// last token precedes i - w.
__device__ __forceinline__ int n_candidates(long i, int window, int cell, int n_cells) {
    if (i < window) return 0;
    long n = (i - window) / cell;
    return (int)(n < n_cells ? n : n_cells);
}

}  // namespace fs
