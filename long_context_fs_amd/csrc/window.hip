// window.hip -- local RoPE branch (FreeSolo summary, section 3.2, eqs. 3-4).
//
// Eq. 3's right-hand side, q_i . R(j - i) k_j, depends on positions only through
// j - i.  The kernels therefore rotate by relative offsets taken from a cos/sin
// table built in fp64 (then rounded to fp32) for offsets -w-128 .. 127.  No
// absolute angle i * theta is ever formed in fp32, so accuracy does not decay
// at 256k positions.
#include "fs_device.hpp"
#include "fs_launch.hpp"

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

hipError_t launch_window(const Shape& sh, const void* q, const void* k, const void* v,
                         double rope_base, void* table, void* o_sr, hipStream_t st)
{
    if (sh.nq == 0) return hipSuccess;
    const int rows = sh.w + 2 * kTableSlack, half = sh.d / 2;
    const long n_tab = (long)rows * half;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n_tab + 255) / 256)), dim3(256), 0, st,
                       (float2*)table, rows, half, sh.w, log(rope_base));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)sh.d));
    dim3 grid((unsigned)((sh.nq + 3) / 4), (unsigned)(sh.B * sh.H)), block(256);
#define FS_WINDOW(E, D)                                                                          \
    hipLaunchKernelGGL((window_attn_rowwise_kernel<E, D>), grid, block, 0, st,                   \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2],              \
                       (const typename E::storage*)k, (const typename E::storage*)v, sh.kvs[0],  \
                       sh.kvs[1], sh.kvs[2], sh.H, sh.nq, sh.q_pos0, sh.w,                       \
                       (const float2*)table, scale_log2, (typename E::storage*)o_sr, sh.os[0],   \
                       sh.os[1], sh.os[2])
    if (sh.bf16) {
        if (sh.d == 64) FS_WINDOW(Bf16, 64); else FS_WINDOW(Bf16, 128);
    } else {
        if (sh.d == 64) FS_WINDOW(F32, 64); else FS_WINDOW(F32, 128);
    }
#undef FS_WINDOW
    return hipGetLastError();
}

}  // namespace fs
