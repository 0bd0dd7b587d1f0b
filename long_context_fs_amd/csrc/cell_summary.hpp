// cell_summary.hpp -- one cell's summaries of eq. 5 (FreeSolo summary, section
// 3.3): the mean key kbar_c and the largest token-key norm a_c, computed by one
// wavefront.  Shared by the batch summaries and the streaming state, so both
// give bit-identical values for the same keys.
#pragma once

#include "fs_device.hpp"

namespace fs {

// The cell's 32 key rows start at row0 and are kvs2 elements apart.  They are
// read with 16-byte loads, several tokens per wave-load.  Each lane keeps a
// running sum of its d-slice (the mean is a register sum) and one squared norm
// per token it touched; a token's norm is finished by a butterfly over the lanes
// that share the token, then a max over tokens.  kbar_out[0..D) (16-byte
// aligned) is written by the lanes of the first token row, *amax_out by lane 0.
// STREAM: the keys are read once (non-temporal loads, bf16 storage).
template <class E, int D, bool STREAM = false>
__device__ __forceinline__ void wave_cell_summary(const typename E::storage* __restrict__ row0,
                                                  int64_t kvs2, float* kbar_out, float* amax_out)
{
    constexpr int EPL = E::kPer16B;   // elements per 16-byte lane load
    constexpr int L = D / EPL;        // lanes per token row
    constexpr int TPL = kWave / L;    // tokens per wave-load
    constexpr int LOADS = 32 / TPL;   // wave-loads per cell
    static_assert(LOADS * TPL == 32, "cell of 32 tokens");

    const int lane = threadIdx.x & 63;
    const int t0 = lane / L, ch = lane % L;
    const typename E::storage* base = row0 + (int64_t)t0 * kvs2 + ch * EPL;

    float x[LOADS][EPL];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        const typename E::storage* p = base + (int64_t)(it * TPL) * kvs2;
        if constexpr (STREAM && EPL == 8) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[it][2 * i] = __uint_as_float(w[i] << 16);
                x[it][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else {
            load16<E>(p, x[it]);
        }
    }

    float sum[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = 0.f;
    float best = 0.f;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            sum[e] += x[it][e];
            sq = fmaf(x[it][e], x[it][e], sq);
        }
#pragma unroll
        for (int m = 1; m < L; m <<= 1) sq += __shfl_xor(sq, m, kWave);
        best = fmaxf(best, sq);
    }
#pragma unroll
    for (int m = L; m < kWave; m <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sum[e] += __shfl_xor(sum[e], m, kWave);
        best = fmaxf(best, __shfl_xor(best, m, kWave));
    }
    if (t0 == 0) {
        float* dst = kbar_out + ch * EPL;            // 16-byte aligned: D % 4 == 0
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(sum[e] * (1.f / 32), sum[e + 1] * (1.f / 32), sum[e + 2] * (1.f / 32),
                            sum[e + 3] * (1.f / 32));
    }
    if (lane == 0) *amax_out = sqrtf(best);
}

}  // namespace fs
