// summaries.hip -- cell summaries (FreeSolo summary, section 3.3, eq. 5).
//
// One wavefront per 32-token cell.  The cell's keys (32 rows of d elements) are
// read with 16-byte loads, several tokens per wave-load, so a wave streams the
// cell in 4-16 fully coalesced loads issued back to back.  Each lane keeps a
// running sum of its d-slice (the mean is a register sum) and one squared norm
// per token it touched; the token norm is finished by a butterfly over the
// lanes that share the token, then a max over tokens.  HBM-bound: every key
// byte is read once, kbar (fp32) and amax are written once.
#include "fs_device.hpp"
#include "fs_launch.hpp"

namespace fs {

template <class E, int D>
__global__ __launch_bounds__(256) void cell_summaries_kernel(
    const typename E::storage* __restrict__ k, int64_t kvs0, int64_t kvs1, int64_t kvs2, int H,
    int C, long total, float* __restrict__ kbar, float* __restrict__ amax)
{
    constexpr int EPL = E::kPer16B;   // elements per 16-byte lane load
    constexpr int L = D / EPL;        // lanes per token row
    constexpr int TPL = kWave / L;    // tokens per wave-load
    constexpr int LOADS = 32 / TPL;   // wave-loads per cell
    static_assert(LOADS * TPL == 32, "cell of 32 tokens");

    const long cell_id = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (cell_id >= total) return;
    const int lane = threadIdx.x & 63;
    const int c = (int)(cell_id % C);
    const long bh = cell_id / C;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int t0 = lane / L, ch = lane % L;
    const typename E::storage* base =
        k + b * kvs0 + h * kvs1 + (int64_t)(c * 32 + t0) * kvs2 + ch * EPL;

    float x[LOADS][EPL];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) load16<E>(base + (int64_t)(it * TPL) * kvs2, x[it]);

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
        float* dst = kbar + (bh * C + c) * (long)D + ch * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(sum[e] * (1.f / 32), sum[e + 1] * (1.f / 32), sum[e + 2] * (1.f / 32),
                            sum[e + 3] * (1.f / 32));
    }
    if (lane == 0) amax[bh * C + c] = sqrtf(best);
}

hipError_t launch_summaries(const Shape& sh, const void* k, float* kbar, float* amax,
                            hipStream_t st)
{
    const long total = (long)sh.B * sh.H * sh.C;
    if (total == 0) return hipSuccess;
    dim3 grid((unsigned)((total + 3) / 4)), block(256);
#define FS_SUMMARIES(E, D)                                                                     \
    hipLaunchKernelGGL((cell_summaries_kernel<E, D>), grid, block, 0, st,                      \
                       (const typename E::storage*)k, sh.kvs[0], sh.kvs[1], sh.kvs[2], sh.H,  \
                       sh.C, total, kbar, amax)
    if (sh.bf16) {
        if (sh.d == 64) FS_SUMMARIES(Bf16, 64); else FS_SUMMARIES(Bf16, 128);
    } else {
        if (sh.d == 64) FS_SUMMARIES(F32, 64); else FS_SUMMARIES(F32, 128);
    }
#undef FS_SUMMARIES
    return hipGetLastError();
}

}  // namespace fs
