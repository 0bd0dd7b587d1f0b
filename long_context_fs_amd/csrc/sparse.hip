// sparse.hip -- long-range token readout with RMSNorm (FreeSolo summary,
// section 3.3, eq. 9).
//
// u_i = softmax over the tokens of the selected cells of q_i . k_j / sqrt(d)
// (unrotated, NoPE), times v_j; o_lr_i = u_i / sqrt(mean(u_i^2) + eps).
#include "fs_device.hpp"
#include "fs_launch.hpp"

namespace fs {

// One wavefront per query row; lanes take two selected cells (64 tokens) at a time.
template <class E, int D>
__global__ __launch_bounds__(256) void sparse_attn_rowwise_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const typename E::storage* __restrict__ k, const typename E::storage* __restrict__ v,
    int64_t kvs0, int64_t kvs1, int64_t kvs2, int H, int nq, const int32_t* __restrict__ idx,
    int topk, float scale_log2, float rms_eps, typename E::storage* __restrict__ o,
    int64_t os0, int64_t os1, int64_t os2)
{
    constexpr int EPL = E::kPer16B;
    constexpr int R = D / kWave;
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

    const int32_t* sel = idx + (bh * nq + row) * (long)topk;
    int n_sel = 0;
    for (int a0 = 0; a0 < topk; a0 += kWave) {
        const bool ok = a0 + lane < topk && sel[a0 + lane] >= 0;
        n_sel += __popcll(__ballot(ok));
    }
    const typename E::storage* kh = k + b * kvs0 + h * kvs1;
    const typename E::storage* vh = v + b * kvs0 + h * kvs1;
    const float* qv = s_q[wv];

    float m = -INFINITY, l = 0.f, acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    for (int a0 = 0; a0 < n_sel; a0 += 2) {
        const int a = a0 + (lane >> 5);
        const bool valid = a < n_sel;
        long j = 0;
        float s = -INFINITY;
        if (valid) {
            j = (long)sel[a] * 32 + (lane & 31);
            const typename E::storage* kr = kh + j * kvs2;
            float dot = 0.f;
            for (int e0 = 0; e0 < D; e0 += EPL) {
                float x[EPL];
                load16<E>(kr + e0, x);
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e0 + e], x[e], dot);
            }
            s = dot * scale_log2;
        }
        const float m_new = fmaxf(m, wave_max(s));
        const float corr = exp2f(m - m_new);
        const float p = valid ? exp2f(s - m_new) : 0.f;
        l = l * corr + wave_sum(p);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] *= corr;
        const int cnt = (n_sel - a0) >= 2 ? kWave : 32;
        for (int jj = 0; jj < cnt; ++jj) {
            const float pj = __shfl(p, jj, kWave);
            const long jt = (long)sel[a0 + (jj >> 5)] * 32 + (jj & 31);
            const typename E::storage* vr = vh + jt * kvs2;
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = fmaf(pj, load1<E>(vr + lane + r * kWave), acc[r]);
        }
        m = m_new;
    }
    float u[R], ss = 0.f;
    const float inv_l = n_sel > 0 ? 1.f / l : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        u[r] = acc[r] * inv_l;
        ss = fmaf(u[r], u[r], ss);
    }
    ss = wave_sum(ss);
    const float inv_rms = 1.f / sqrtf(ss / (float)D + rms_eps);
    typename E::storage* orow = o + b * os0 + h * os1 + row * os2;
#pragma unroll
    for (int r = 0; r < R; ++r) store1<E>(orow + lane + r * kWave, u[r] * inv_rms);
}

hipError_t launch_sparse(const Shape& sh, const void* q, const void* k, const void* v,
                         const int32_t* idx, int topk, float rms_eps, void* o_lr, hipStream_t st)
{
    if (sh.nq == 0) return hipSuccess;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)sh.d));
    dim3 grid((unsigned)((sh.nq + 3) / 4), (unsigned)(sh.B * sh.H)), block(256);
#define FS_SPARSE(E, D)                                                                          \
    hipLaunchKernelGGL((sparse_attn_rowwise_kernel<E, D>), grid, block, 0, st,                   \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2],              \
                       (const typename E::storage*)k, (const typename E::storage*)v, sh.kvs[0],  \
                       sh.kvs[1], sh.kvs[2], sh.H, sh.nq, idx, topk, scale_log2, rms_eps,        \
                       (typename E::storage*)o_lr, sh.os[0], sh.os[1], sh.os[2])
    if (sh.bf16) {
        if (sh.d == 64) FS_SPARSE(Bf16, 64); else FS_SPARSE(Bf16, 128);
    } else {
        if (sh.d == 64) FS_SPARSE(F32, 64); else FS_SPARSE(F32, 128);
    }
#undef FS_SPARSE
    return hipGetLastError();
}

}  // namespace fs
