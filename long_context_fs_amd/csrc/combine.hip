// combine.hip -- range separation (FreeSolo summary, section 3.1, eq. 2):
// o_i = o_sr_i + alpha_h * o_lr_i.  Elementwise and HBM-bound: 16-byte loads
// (non-temporal for bf16) and stores, one vector per thread.
#include "fs_device.hpp"
#include "fs_launch.hpp"

namespace fs {

template <class E, int D>
__global__ __launch_bounds__(256) void combine_kernel(
    const typename E::storage* __restrict__ o_sr, const typename E::storage* __restrict__ o_lr,
    typename E::storage* __restrict__ o, int64_t os0, int64_t os1, int64_t os2, int H, int nq,
    long total_vec, const float* __restrict__ alpha)
{
    constexpr int EPL = E::kPer16B;
    constexpr int VPR = D / EPL;       // vectors per row
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total_vec) return;
    const int e0 = (int)(t % VPR) * EPL;
    const long rowid = t / VPR;
    const long row = rowid % nq;
    const long bh = rowid / nq;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int64_t off = b * os0 + h * os1 + row * os2 + e0;
    const float a = alpha[h];
    float x[EPL], y[EPL], z[EPL];
    if constexpr (EPL == 8) {          // bf16: both branch outputs are read once
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 wx = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_sr + off));
        const u32x4 wy = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_lr + off));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(wx[i] << 16);
            x[2 * i + 1] = __uint_as_float(wx[i] & 0xFFFF0000u);
            y[2 * i] = __uint_as_float(wy[i] << 16);
            y[2 * i + 1] = __uint_as_float(wy[i] & 0xFFFF0000u);
        }
    } else {
        load16<E>(o_sr + off, x);
        load16<E>(o_lr + off, y);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) z[e] = fmaf(a, y[e], x[e]);
    store16<E>(o + off, z);
}

hipError_t launch_combine(const Shape& sh, const void* o_sr, const void* o_lr, const float* alpha,
                          void* o, hipStream_t st)
{
    const long total_vec = (long)sh.B * sh.H * sh.nq * (sh.d / (sh.bf16 ? 8 : 4));
    if (total_vec == 0) return hipSuccess;
    dim3 grid((unsigned)((total_vec + 255) / 256)), block(256);
#define FS_COMBINE(E, D)                                                                         \
    hipLaunchKernelGGL((combine_kernel<E, D>), grid, block, 0, st,                               \
                       (const typename E::storage*)o_sr, (const typename E::storage*)o_lr,       \
                       (typename E::storage*)o, sh.os[0], sh.os[1], sh.os[2], sh.H, sh.nq,       \
                       total_vec, alpha)
    if (sh.bf16) {
        if (sh.d == 64) FS_COMBINE(Bf16, 64); else FS_COMBINE(Bf16, 128);
    } else {
        if (sh.d == 64) FS_COMBINE(F32, 64); else FS_COMBINE(F32, 128);
    }
#undef FS_COMBINE
    return hipGetLastError();
}

}  // namespace fs
