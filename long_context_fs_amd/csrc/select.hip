// select.hip -- cell scoring and per-query top-K (FreeSolo summary, section 3.3,
// eq. 7 with lambda_h = 0; the selected set S_i of eq. 9).
//
// One wavefront per query row.  The unrotated query is staged in LDS; each lane
// scores candidate cells c (from the keep row of the query's candidate count,
// or every c < n_i without pruning) as the fp32 dot q . kbar_c.  Ranking uses
// the unscaled dot (1/sqrt(d) > 0 does not change the order and must not merge
// neighbouring scores); the reported score is dot / sqrt(d).  The K-th largest
// key is found exactly by a bitwise search with ballot counts, ties at the
// threshold go to the larger cell, and the chosen cells are written ascending.
#include "fs_device.hpp"
#include "fs_launch.hpp"

namespace fs {

constexpr int kSelWaves = 4;

__device__ __forceinline__ float key_to_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <class E, int D>
__global__ __launch_bounds__(kSelWaves * kWave) void select_topk_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const float* __restrict__ kbar, int H, int C, int nq, int q_pos0, int window, int cell,
    const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_count, int keep_w,
    int n_lo, int n_rows, int topk, int cap, float inv_sqrt_d, int32_t* __restrict__ idx,
    float* __restrict__ score)
{
    extern __shared__ uint32_t smem[];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    float* s_q = reinterpret_cast<float*>(smem) + wv * D;
    uint32_t* s_key = smem + waves * D + wv * cap;

    const long row = (long)blockIdx.x * waves + wv;
    const long bh = blockIdx.y;
    const bool active = row < nq;       // inactive waves still reach the barrier
    const int h = (int)(bh % H), b = (int)(bh / H);
    const long i = (long)q_pos0 + (active ? row : 0);
    const int n = active ? n_candidates(i, window, cell, C) : 0;

    const int32_t* cand = nullptr;
    int n_cand = n;
    if (keep != nullptr) {
        n_cand = 0;
        if (n > 0) {
            const long kr = bh * n_rows + (n - n_lo);
            cand = keep + kr * keep_w;
            n_cand = keep_count[kr];
        }
    }
    if (active) {
        const typename E::storage* qrow = q + b * qs0 + h * qs1 + row * qs2;
        for (int e = lane; e < D; e += kWave) s_q[e] = load1<E>(qrow + e);
    }
    __syncthreads();

    const float* kb_head = kbar + bh * (long)C * D;
    for (int j = lane; j < n_cand; j += kWave) {
        const int c = cand ? cand[j] : j;
        const float* kb = kb_head + (long)c * D;
        float dot = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; e += 4) {
            const float4 kv = *reinterpret_cast<const float4*>(kb + e);
            dot = fmaf(s_q[e], kv.x, dot);
            dot = fmaf(s_q[e + 1], kv.y, dot);
            dot = fmaf(s_q[e + 2], kv.z, dot);
            dot = fmaf(s_q[e + 3], kv.w, dot);
        }
        s_key[j] = float_key(dot);
    }
    __syncthreads();
    if (!active) return;

    const int kq = n_cand < topk ? n_cand : topk;
    uint32_t thr = 0;
    if (kq > 0) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t t = thr | (1u << bit);
            int cnt = 0;
            for (int j = lane; j < n_cand; j += kWave) cnt += s_key[j] >= t;
            if (wave_sum_int(cnt) >= kq) thr = t;
        }
    }
    int n_gt = 0, n_eq = 0;
    for (int j = lane; j < n_cand; j += kWave) {
        n_gt += s_key[j] > thr;
        n_eq += s_key[j] == thr;
    }
    n_gt = wave_sum_int(n_gt);
    n_eq = wave_sum_int(n_eq);
    const int need_eq = kq - n_gt;

    int32_t* out_i = idx + (bh * nq + row) * (long)topk;
    float* out_s = score ? score + (bh * nq + row) * (long)topk : nullptr;
    int written = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n_cand && kq > 0; j0 += kWave) {
        const int j = j0 + lane;
        const bool in = j < n_cand;
        const uint32_t kj = in ? s_key[j] : 0u;
        const bool is_eq = in && kj == thr;
        const uint64_t me = __ballot(is_eq);
        const int eq_rank = eq_seen + lanes_below(me);
        const bool kept = in && (kj > thr || (is_eq && eq_rank >= n_eq - need_eq));
        const uint64_t mk = __ballot(kept);
        if (kept) {
            const int pos = written + lanes_below(mk);
            out_i[pos] = cand ? cand[j] : j;
            if (out_s) out_s[pos] = key_to_float(kj) * inv_sqrt_d;
        }
        written += __popcll(mk);
        eq_seen += __popcll(me);
    }
    for (int t = kq + lane; t < topk; t += kWave) {
        out_i[t] = -1;
        if (out_s) out_s[t] = 0.f;
    }
}

hipError_t launch_select(const Shape& sh, const void* q, const float* kbar, const int32_t* keep,
                         const int32_t* keep_count, int keep_w, int n_lo, int n_rows, int topk,
                         int32_t* idx, float* score, hipStream_t st)
{
    if (sh.nq == 0) return hipSuccess;
    // Largest candidate list: the keep width, or every cell below the last query's n.
    int n_hi = 0;
    {
        long i = (long)sh.q_pos0 + sh.nq - 1;
        if (i >= sh.w) n_hi = (int)((i - sh.w) / sh.s);
        if (n_hi > sh.C) n_hi = sh.C;
    }
    const int cap = keep ? keep_w : (n_hi > 0 ? n_hi : 1);
    // As many waves (query rows) per block as fit in 64 KiB of LDS.
    int waves = kSelWaves;
    while (waves > 1 && (size_t)waves * (sh.d + cap) * sizeof(uint32_t) > 65536) waves >>= 1;
    const size_t lds = (size_t)waves * (sh.d + cap) * sizeof(uint32_t);
    if (lds > 65536) return hipErrorInvalidValue;
    dim3 grid((unsigned)((sh.nq + waves - 1) / waves), (unsigned)(sh.B * sh.H));
    dim3 block(waves * kWave);
    const float inv_sqrt_d = 1.0f / sqrtf((float)sh.d);
#define FS_SELECT(E, D)                                                                        \
    hipLaunchKernelGGL((select_topk_kernel<E, D>), grid, block, lds, st,                       \
                       (const typename E::storage*)q, sh.qs[0], sh.qs[1], sh.qs[2], kbar, sh.H, \
                       sh.C, sh.nq, sh.q_pos0, sh.w, sh.s, keep, keep_count, keep_w, n_lo,      \
                       n_rows, topk, cap, inv_sqrt_d, idx, score)
    if (sh.bf16) {
        if (sh.d == 64) FS_SELECT(Bf16, 64); else FS_SELECT(Bf16, 128);
    } else {
        if (sh.d == 64) FS_SELECT(F32, 64); else FS_SELECT(F32, 128);
    }
#undef FS_SELECT
    return hipGetLastError();
}

}  // namespace fs
