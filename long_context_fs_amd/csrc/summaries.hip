// summaries.hip -- cell summaries (FreeSolo summary, section 3.3, eq. 5).
//
// One wavefront per 32-token cell.  The cell's keys (32 rows of d elements) are
// read with 16-byte loads, several tokens per wave-load, so a wave streams the
// cell in 4-16 fully coalesced loads issued back to back.  Each lane keeps a
// running sum of its d-slice (the mean is a register sum) and one squared norm
// per token it touched; the token norm is finished by a butterfly over the
// lanes that share the token, then a max over tokens.  HBM-bound: every key
// byte is read once (non-temporal loads for bf16 keys), kbar (fp32) and amax
// are written once.
#include "cell_summary.hpp"
#include "fs_device.hpp"
#include "fs_launch.hpp"

namespace fs {

template <class E, int D>
__global__ __launch_bounds__(256) void cell_summaries_kernel(
    const typename E::storage* __restrict__ k, int64_t kvs0, int64_t kvs1, int64_t kvs2, int H,
    int C, long total, float* __restrict__ kbar, float* __restrict__ amax)
{
    const long cell_id = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (cell_id >= total) return;
    const int c = (int)(cell_id % C);
    const long bh = cell_id / C;
    const int h = (int)(bh % H), b = (int)(bh / H);
    wave_cell_summary<E, D, true>(k + b * kvs0 + h * kvs1 + (int64_t)c * 32 * kvs2, kvs2,
                                  kbar + (bh * C + c) * (long)D, amax + bh * C + c);
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
