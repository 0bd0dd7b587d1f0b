// fsb.hip -- FS-B balanced tree search (FreeSolo summary, section 3.4, eqs. 10-11).
//
// Forests.  A causal forest over a sequence of cells is the set of complete,
// aligned power-of-two blocks of the sequence: node (l, j) covers leaves
// j 2^l .. (j+1) 2^l - 1, its children are (l-1, 2j) and (l-1, 2j+1), and a
// prefix of n leaves is covered by one root per set bit of n.  Forest 0 holds
// every complete cell (A^0 = C_i); a forest with thresholds tau_h holds the
// cells with a_c >= tau_h in ascending order (A^tau, eq. 10).  Node statistics:
// mu_v the mean of its cell means (fp64 sum in ascending leaf order, scaled by
// 2^-l, rounded to fp32), rho_v the largest distance from mu_v to one of them
// (fp64, rounded to fp32), A_v the largest a_c, p_v^min the centre of its first
// cell.  Built by three kernels: admission (a block scan per head), means (a
// thread per (node, dim)), radii (a thread per (level, leaf)).
//
// Search.  One wave per (query, head) searches both forests in turn; in each the
// beam starts from the best B
// roots, each step replaces inner nodes by their children, keeps leaves and
// retains the best B by U_v = (q.mu_v + c |q| rho_v) / sqrt(d) + lambda_h A_v
// erf((i - p_v^min) / (2 sigma_h)) (eq. 11), until only leaves remain.  S_i is
// the best min(K, #found) cells of the two final beams by that score (a leaf's
// U is eq. 7's r_ic).  The search decides by comparing U, so U is computed in
// one fixed order: fp64 on the fp32 statistics, dot products as 16 partial
// sums over contiguous d/16-element chunks added pairwise at distances 8, 4, 2,
// 1 (a butterfly's result at position 0).  Four lanes score one node, 16 nodes
// per pass: lane r sums chunks r, r+4, r+8, r+12 and does the first two pair
// levels in registers, the last two by shuffles.  Ties: the
// larger U, then the later block, then the lower level.  Floating-point
// contraction is off in this file so every product and sum rounds on its own.
//
// Reranking (eq. 12, section 3.4).  Given the raw keys, the found cells are
// ranked instead by r~ = log sum_j exp(q.k_j / sqrt(d)) over the cell's s = 32
// keys plus the prior at the cell: a half-wave per cell, one key per lane (an
// fp32 dot product in ascending element order), the half-wave's maximum and
// sum of exp2 by shuffles.
#include <cmath>

#include "fs_device.hpp"
#include "fs_launch.hpp"

#pragma clang fp contract(off)

namespace fs {

namespace {

constexpr int kMaxBeam = 64;
constexpr int kMaxLevels = 16;

struct FsbLayout {
    int C, d, n_levels;
    int lev_off[kMaxLevels + 1];   // node index of (l, 0); lev_off[n_levels] = nodes
    int64_t off_prefix, off_first, off_amax, off_rho, off_mu, stride;
};

FsbLayout fsb_layout(int C, int d)
{
    FsbLayout L{};
    L.C = C;
    L.d = d;
    int lv = 0, nodes = 0;
    while (lv < kMaxLevels && (C >> lv) > 0) {
        L.lev_off[lv] = nodes;
        nodes += C >> lv;
        ++lv;
    }
    L.n_levels = lv;
    for (int l = lv; l <= kMaxLevels; ++l) L.lev_off[l] = nodes;
    auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
    int64_t off = 256;   // int32 leaf count m at byte 0
    L.off_prefix = off;
    off = up(off + 4 * (int64_t)(C + 1));
    L.off_first = off;
    off = up(off + 4 * (int64_t)nodes);
    L.off_amax = off;
    off = up(off + 4 * (int64_t)nodes);
    L.off_rho = off;
    off = up(off + 4 * (int64_t)nodes);
    L.off_mu = off;
    off = up(off + 4 * (int64_t)nodes * d);
    L.stride = off;
    return L;
}

struct FsbView {
    int* m;
    int* prefix;
    int* first;
    float* amax;
    float* rho;
    float* mu;
};

__device__ __forceinline__ FsbView fsb_view(char* base, const FsbLayout& L, long bh)
{
    char* F = base + bh * L.stride;
    return FsbView{reinterpret_cast<int*>(F), reinterpret_cast<int*>(F + L.off_prefix),
                   reinterpret_cast<int*>(F + L.off_first), reinterpret_cast<float*>(F + L.off_amax),
                   reinterpret_cast<float*>(F + L.off_rho), reinterpret_cast<float*>(F + L.off_mu)};
}

__device__ __forceinline__ int fsb_level_of(const FsbLayout& L, int node)
{
    int l = 0;
    while (l + 1 < L.n_levels && L.lev_off[l + 1] <= node) ++l;
    return l;
}

// ---- forest construction ----------------------------------------------------

// Admission (eq. 10) and the leaf order: one block per (b, h) scans the cells.
__global__ __launch_bounds__(256) void forest_admit_kernel(const float* __restrict__ amax,
                                                           const float* __restrict__ tau, int H,
                                                           FsbLayout L, char* __restrict__ forest)
{
    const long bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const FsbView f = fsb_view(forest, L, bh);
    const float* a = amax + bh * L.C;
    const float th = tau ? tau[bh % H] : 0.f;
    __shared__ int wsum[4];
    int base = 0;
    if (tid == 0) f.prefix[0] = 0;
    for (int c0 = 0; c0 < L.C; c0 += 256) {
        const int c = c0 + tid;
        const bool in = c < L.C && (!tau || a[c] >= th);
        const uint64_t bal = __ballot(in);
        const int below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[wv] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            before += w < wv ? wsum[w] : 0;
            total += wsum[w];
        }
        const int pos = base + before + below;
        if (in) f.first[pos] = c;                 // leaf pos is node (0, pos)
        if (c < L.C) f.prefix[c + 1] = pos + (in ? 1 : 0);
        base += total;
        __syncthreads();
    }
    if (tid == 0) *f.m = base;
}

// mu_v, A_v and the first cell of every node: a thread per (node, dim).
__global__ __launch_bounds__(256) void forest_mean_kernel(const float* __restrict__ kbar,
                                                          const float* __restrict__ amax,
                                                          FsbLayout L, char* __restrict__ forest)
{
    const long bh = blockIdx.y;
    const int per = 256 / L.d;
    const int nodes = L.lev_off[L.n_levels];
    // top levels first: their long serial sums start with the first blocks
    const int node = nodes - 1 - (blockIdx.x * per + threadIdx.x / L.d), e = threadIdx.x % L.d;
    if (node < 0) return;
    const FsbView f = fsb_view(forest, L, bh);
    const int l = fsb_level_of(L, node), j = node - L.lev_off[l];
    if (j >= (*f.m >> l)) return;
    const int leaf0 = j << l, width = 1 << l;
    const float* kb = kbar + bh * (long)L.C * L.d;
    const float* a = amax + bh * (long)L.C;
    double s = 0.0;
    float a_best = -INFINITY;
    int t = 0;
    // 32 leaves per round, the next round's cell indices loaded with this round's
    // values; the sum still runs in ascending leaf order (leaf0 is a multiple of
    // 32 here)
    if (width >= 32) {
        const int4* c4 = reinterpret_cast<const int4*>(f.first + leaf0);
        int4 cur[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cur[u] = c4[u];
        for (; t + 32 <= width; t += 32) {
            float x[32], av[32];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int cc[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    x[4 * u + w] = kb[(long)cc[w] * L.d + e];
                    av[4 * u + w] = a[cc[w]];
                }
            }
            if (t + 64 <= width) {
#pragma unroll
                for (int u = 0; u < 8; ++u) cur[u] = c4[(t + 32) / 4 + u];
            }
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                s += (double)x[u];
                if (av[u] > a_best) a_best = av[u];
            }
        }
    }
    for (; t < width; ++t) {
        const int c = f.first[leaf0 + t];
        s += (double)kb[(long)c * L.d + e];
        if (a[c] > a_best) a_best = a[c];
    }
    f.mu[(long)node * L.d + e] = (float)(s * __builtin_ldexp(1.0, -l));
    if (e == 0) {
        f.amax[node] = a_best;
        f.rho[node] = 0.f;
        if (l > 0) f.first[node] = f.first[leaf0];
    }
}

// rho_v: a thread per (level, leaf) computes the leaf's squared distance to its
// node's mean (summed over d in order, fp64), a segmented wave maximum combines
// the node's leaves, and nodes wider than a wave combine their waves with an
// integer maximum on the fp32 bits of sqrt(max) (rho >= 0, and rounding and sqrt
// are monotone, so this equals rounding the square root of the overall maximum).
// forest_mean_kernel zeroes rho first.
template <int D>
__global__ __launch_bounds__(256) void forest_radius_kernel(const float* __restrict__ kbar,
                                                            FsbLayout L, char* __restrict__ forest)
{
    const long bh = blockIdx.z;
    const int l = blockIdx.y, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 256 + threadIdx.x;
    const FsbView f = fsb_view(forest, L, bh);
    const int n_nodes = *f.m >> l, j = t >> l;
    const bool on = j < n_nodes;
    double r2 = 0.0;
    if (on) {
        const float4* kr = reinterpret_cast<const float4*>(kbar + (bh * (long)L.C + f.first[t]) * D);
        const float4* mu = reinterpret_cast<const float4*>(f.mu + (long)(L.lev_off[l] + j) * D);
#pragma unroll 8
        for (int g = 0; g < D / 4; ++g) {
            const float4 a = kr[g], m = mu[g];
            double diff = (double)a.x - (double)m.x;
            r2 = __builtin_fma(diff, diff, r2);
            diff = (double)a.y - (double)m.y;
            r2 = __builtin_fma(diff, diff, r2);
            diff = (double)a.z - (double)m.z;
            r2 = __builtin_fma(diff, diff, r2);
            diff = (double)a.w - (double)m.w;
            r2 = __builtin_fma(diff, diff, r2);
        }
    }
    const int seg = l < 6 ? 1 << l : kWave;       // lanes holding one node's leaves
    for (int off = seg >> 1; off >= 1; off >>= 1) {
        const double o = __shfl_xor(r2, off);
        if (o > r2) r2 = o;
    }
    if (on && (lane & (seg - 1)) == 0) {
        const float rho = (float)__builtin_sqrt(r2);
        atomicMax(reinterpret_cast<int*>(f.rho + L.lev_off[l] + j), __float_as_int(rho));
    }
}

// ---- search -------------------------------------------------------------------

// Per-wave search state in LDS, kept small (cells and node indices < 32768 fit
// int16) so that many waves fit a compute unit.
struct BeamLds {
    alignas(16) float q[128];     // the query row
    double cu[2 * kMaxBeam];      // candidates: U, level, index, first cell
    double bu[kMaxBeam];          // the beam
    double fu[2 * kMaxBeam];      // leaves found by both forests: score, cell
    int16_t cix[2 * kMaxBeam], cfirst[2 * kMaxBeam];
    int16_t bix[kMaxBeam], bfirst[kMaxBeam];
    int16_t fcell[2 * kMaxBeam];
    int16_t fleaf[2 * kMaxBeam];  // the found cell's leaf index in its forest
    uint8_t clv[2 * kMaxBeam], blv[kMaxBeam];
    uint8_t todo[2 * kMaxBeam];   // candidate slots whose U is still to be computed
    uint8_t fdup[2 * kMaxBeam];   // found twice (second forest)
    uint8_t frank[2 * kMaxBeam];  // rank among the found cells
    int ctie[2 * kMaxBeam];       // candidates' tie order
};

struct QueryCtx {
    const float4* q;              // the query row in LDS
    double q_norm;
    double i_pos;                 // the query's position
    double lam, sig;              // eq. 7 prior of the head (lam 0: none)
    double slack, inv_sqrt_d;
    int s;
};

// Lane r's share of q . x: chunks r, r+4, r+8, r+12 (D/16 elements each, fma in
// ascending order), combined as (p_r + p_{r+8}) + (p_{r+4} + p_{r+12}).  Two
// shuffles at distances 2 and 1 then finish the pairwise sum.
template <int D>
__device__ __forceinline__ double dot_share(const float4* q, const float4* x4, int r)
{
    constexpr int C4 = D / 64;
    float4 xv4[4][C4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < C4; ++g) xv4[j][g] = x4[(r + 4 * j) * C4 + g];
    double p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        double acc = 0.0;
#pragma unroll
        for (int g = 0; g < C4; ++g) {
            const float4 xv = xv4[j][g], qv = q[(r + 4 * j) * C4 + g];
            acc = __builtin_fma((double)qv.x, (double)xv.x, acc);
            acc = __builtin_fma((double)qv.y, (double)xv.y, acc);
            acc = __builtin_fma((double)qv.z, (double)xv.z, acc);
            acc = __builtin_fma((double)qv.w, (double)xv.w, acc);
        }
        p[j] = acc;
    }
    return (p[0] + p[2]) + (p[1] + p[3]);
}

__device__ __forceinline__ double dot_finish(double part)
{
    part = part + __shfl_xor(part, 2);
    return part + __shfl_xor(part, 1);
}

__device__ __forceinline__ bool beam_better(double ub, int fb, int lb, double ua, int fa, int la)
{
    return ub > ua || (ub == ua && (fb > fa || (fb == fa && lb < la)));
}

// lambda_h A_v erf((i - p) / (2 sigma_h)), kept out of line so that erf's
// registers do not weigh on the search without a prior.
__device__ __attribute__((noinline)) double fsb_prior(double lam, double a_v, double i_pos,
                                                       double p_c, double sig)
{
    return lam * a_v * erf((i_pos - p_c) / (2.0 * sig));
}

// U of the candidates listed in todo[0 .. n_todo): four lanes per node.
template <int D>
__device__ __forceinline__ void beam_score(BeamLds& S, int n_todo, const FsbView& f,
                                           const FsbLayout& L, const QueryCtx& Q)
{
    const int lane = threadIdx.x & 63, r = lane & 3;
    for (int k0 = 0; k0 < n_todo; k0 += 16) {
        const int k = k0 + (lane >> 2);
        const bool valid = k < n_todo;
        int slot = 0, node = 0, c = 0;
        float rho = 0.f, a_v = 0.f;
        double part = 0.0;
        if (valid) {
            slot = S.todo[k];
            node = L.lev_off[S.clv[slot]] + S.cix[slot];
            // the node's statistics load alongside its mean row
            if (r == 0) {
                rho = f.rho[node];
                c = f.first[node];
                a_v = f.amax[node];
            }
            part = dot_share<D>(Q.q, reinterpret_cast<const float4*>(f.mu + (long)node * D), r);
        }
        const double dot = dot_finish(part);
        if (valid && r == 0) {
            double t = Q.slack * Q.q_norm;
            t = t * (double)rho;
            double u = dot + t;
            u = u * Q.inv_sqrt_d;
            double prior = 0.0;
            if (Q.lam != 0.0 || Q.sig != 0.0) {
                const double p_c = ((double)c + 0.5) * (double)Q.s;
                prior = fsb_prior(Q.lam, (double)a_v, Q.i_pos, p_c, Q.sig);
            }
            S.cu[slot] = u + prior;
            S.cfirst[slot] = c;
        }
    }
    __syncthreads();
}

// Keeps the best min(n_cand, beam) candidates as the beam; returns its size.
// The tie order (later first cell, then lower level) is one int per candidate,
// first * 16 + 15 - level, so a comparison reads two LDS words.
__device__ __forceinline__ int beam_keep(BeamLds& S, int n_cand, int beam)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = lane + 64 * h;
        if (a < 2 * kMaxBeam) S.ctie[a] = a < n_cand ? S.cfirst[a] * 16 + 15 - S.clv[a] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = lane + 64 * h;
        if (a < n_cand) {
            const double ua = S.cu[a];
            const int la = S.clv[a], ta = S.ctie[a];
            int rank = 0, b = 0;
            for (; b + 4 <= n_cand; b += 4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const double ub = S.cu[b + u];
                    const int tb = S.ctie[b + u];
                    rank += (ub > ua || (ub == ua && tb > ta)) ? 1 : 0;
                }
            }
            for (; b < n_cand; ++b) {
                const double ub = S.cu[b];
                const int tb = S.ctie[b];
                rank += (ub > ua || (ub == ua && tb > ta)) ? 1 : 0;
            }
            if (rank < beam) {
                S.bu[rank] = ua;
                S.blv[rank] = la;
                S.bix[rank] = S.cix[a];
                S.bfirst[rank] = S.cfirst[a];
            }
        }
    }
    __syncthreads();
    return n_cand < beam ? n_cand : beam;
}

// Beam search of one forest over its first n_leaves leaves; appends the final
// beam's cells and scores to the found list at *n_found.
template <int D>
__device__ __forceinline__ void beam_forest(BeamLds& S, const FsbView& f, const FsbLayout& L, int n_leaves,
                            int beam, const QueryCtx& Q, int* n_found, int* n_scored)
{
    const int lane = threadIdx.x & 63;
    if (n_leaves <= 0) return;
    int n_cand = 0, start = 0;
    for (int l = L.n_levels - 1; l >= 0; --l) {
        if ((n_leaves >> l) & 1) {
            if (lane == 0) {
                S.clv[n_cand] = l;
                S.cix[n_cand] = start >> l;
                S.todo[n_cand] = n_cand;
            }
            ++n_cand;
            start += 1 << l;
        }
    }
    __syncthreads();
    beam_score<D>(S, n_cand, f, L, Q);
    *n_scored += n_cand;
    int n_cur = beam_keep(S, n_cand, beam);
    for (;;) {
        const bool inner = lane < n_cur && S.blv[lane] > 0;
        const uint64_t im = __ballot(inner);
        if (im == 0) break;
        const uint64_t below = (1ull << lane) - 1ull;
        if (lane < n_cur) {
            const int pos = lane + __popcll(im & below);
            const int lv = S.blv[lane], ix = S.bix[lane];
            if (!inner) {
                S.cu[pos] = S.bu[lane];
                S.clv[pos] = lv;
                S.cix[pos] = ix;
                S.cfirst[pos] = S.bfirst[lane];
            } else {
                const int r = __popcll(im & below);
                S.clv[pos] = lv - 1;
                S.cix[pos] = 2 * ix;
                S.clv[pos + 1] = lv - 1;
                S.cix[pos + 1] = 2 * ix + 1;
                S.todo[2 * r] = pos;
                S.todo[2 * r + 1] = pos + 1;
            }
        }
        n_cand = n_cur + __popcll(im);
        __syncthreads();
        beam_score<D>(S, 2 * __popcll(im), f, L, Q);
        *n_scored += 2 * __popcll(im);
        n_cur = beam_keep(S, n_cand, beam);
    }
    if (lane < n_cur) {
        S.fu[*n_found + lane] = S.bu[lane];
        S.fcell[*n_found + lane] = S.bfirst[lane];
        S.fleaf[*n_found + lane] = S.bix[lane];
    }
    *n_found += n_cur;
    __syncthreads();
}

// Eq. 12's score of every found cell that is not a repeat, into fu.  kh: the
// head's keys (row stride ks); a0 / at: the leaves' A_v in the forest each
// entry came from (entries below n_first from forest 0).
template <class E, int D>
__device__ __forceinline__ void rerank_found(BeamLds& S, int n_found, int n_first,
                                             const typename E::storage* __restrict__ kh,
                                             int64_t ks, const float* a0, const float* at,
                                             const QueryCtx& Q, float scale_log2)
{
    const int lane = threadIdx.x & 63, j = lane & 31;
    for (int a2 = 0; a2 < n_found; a2 += 2) {
        const int a = a2 + (lane >> 5);
        const bool on = a < n_found && !S.fdup[a];
        float x = -INFINITY;
        if (on) {
            const typename E::storage* kr = kh + ((int64_t)S.fcell[a] * Q.s + j) * ks;
            float acc = 0.f;
#pragma unroll 4
            for (int e0 = 0; e0 < D; e0 += E::kPer16B) {
                float kv[E::kPer16B];
                load16<E>(kr + e0, kv);
#pragma unroll
                for (int t = 0; t < E::kPer16B; ++t) acc = __builtin_fmaf(S.q[e0 + t], kv[t], acc);
            }
            x = acc * scale_log2;
        }
        // xor distances below 32 keep the two half-waves apart
        float m = x;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        float e = on ? exp2f(x - m) : 0.f;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) e += __shfl_xor(e, o);
        if (on && j == 0) {
            double r = (double)((m + log2f(e)) * 0.69314718055994531f);
            if (Q.lam != 0.0 || Q.sig != 0.0) {
                const int c = S.fcell[a];
                const float a_v = (a < n_first ? a0 : at)[S.fleaf[a]];
                r = r + fsb_prior(Q.lam, (double)a_v, Q.i_pos, ((double)c + 0.5) * (double)Q.s,
                                  Q.sig);
            }
            S.fu[a] = r;
        }
    }
    __syncthreads();
}

template <class E, int D, bool RR>
__global__ __launch_bounds__(64, 6) void beam_select_kernel(
    const typename E::storage* __restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
    const typename E::storage* __restrict__ k, int64_t ks0, int64_t ks1, int64_t ks2, int H,
    int nq, int q_pos0, int w, int s, FsbLayout L, char* forest0, char* forest_tau, int beam,
    double slack, double inv_sqrt_d, float scale_log2, const float* __restrict__ prior_lambda,
    const float* __restrict__ prior_sigma, int topk, int32_t* __restrict__ idx,
    float* __restrict__ score, int32_t* __restrict__ effort)
{
    __shared__ BeamLds S;
    const int lane = threadIdx.x;
    const long row = blockIdx.x;
    const long bh = blockIdx.y;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const typename E::storage* qr = q + b * qs0 + h * qs1 + row * qs2;
    for (int e = lane; e < D; e += kWave) S.q[e] = load1<E>(qr + e);
    __syncthreads();
    QueryCtx Q;
    const float4* q4 = reinterpret_cast<const float4*>(S.q);
    Q.q = q4;
    Q.s = s;
    Q.slack = slack;
    Q.inv_sqrt_d = inv_sqrt_d;
    const long i = (long)q_pos0 + row;
    Q.i_pos = (double)i;
    Q.lam = prior_lambda ? (double)prior_lambda[h] : 0.0;
    Q.sig = prior_lambda ? (double)prior_sigma[h] : 0.0;
    Q.q_norm = __builtin_sqrt(dot_finish(dot_share<D>(Q.q, q4, lane & 3)));

    long n = i < w ? 0 : (i - w) / s;
    if (n > L.C) n = L.C;
    int n_found = 0, n_first = 0, n_scored = 0;
    if (forest0) {
        const FsbView f = fsb_view(forest0, L, bh);
        beam_forest<D>(S, f, L, f.prefix[n], beam, Q, &n_found, &n_scored);
    }
    n_first = n_found;
    if (forest_tau) {
        const FsbView f = fsb_view(forest_tau, L, bh);
        beam_forest<D>(S, f, L, f.prefix[n], beam, Q, &n_found, &n_scored);
    }

    // union of the two beams (a cell found twice has the same score), best min(K, .)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int a = lane + 64 * hh;
        if (a < n_found) {
            bool dup = false;
            if (a >= n_first)
                for (int c = 0; c < n_first; ++c) dup |= S.fcell[c] == S.fcell[a];
            S.fdup[a] = dup ? 1 : 0;
        }
    }
    __syncthreads();
    if (RR)
        rerank_found<E, D>(S, n_found, n_first, k + b * ks0 + h * ks1, ks2,
                           forest0 ? fsb_view(forest0, L, bh).amax : nullptr,
                           forest_tau ? fsb_view(forest_tau, L, bh).amax : nullptr, Q, scale_log2);
    int n_unique = 0;
    for (int a = 0; a < n_found; ++a) n_unique += S.fdup[a] ? 0 : 1;
    const int n_sel = n_unique < topk ? n_unique : topk;
    int32_t* orow = idx + (bh * nq + row) * (long)topk;
    float* srow = score ? score + (bh * nq + row) * (long)topk : nullptr;
    // rank by (score, cell) descending, then write the selected cells ascending
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int a = lane + 64 * hh;
        int rank = topk;
        if (a < n_found && !S.fdup[a]) {
            rank = 0;
            for (int c = 0; c < n_found; ++c)
                if (!S.fdup[c]) rank += beam_better(S.fu[c], S.fcell[c], 0, S.fu[a], S.fcell[a], 0);
        }
        S.frank[a] = (uint8_t)rank;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int a = lane + 64 * hh;
        if (a < n_found && S.frank[a] < n_sel) {
            int pos = 0;
            for (int c = 0; c < n_found; ++c)
                pos += (S.frank[c] < n_sel && S.fcell[c] < S.fcell[a]) ? 1 : 0;
            orow[pos] = S.fcell[a];
            if (srow) srow[pos] = (float)S.fu[a];
        }
    }
    if (lane >= n_sel && lane < topk) {
        orow[lane] = -1;
        if (srow) srow[lane] = 0.f;
    }
    if (effort && lane == 0) effort[bh * nq + row] = n_scored;
}

}  // namespace

size_t forest_bytes(const Shape& sh)
{
    return (size_t)fsb_layout(sh.C, sh.d).stride * sh.B * sh.H;
}

hipError_t launch_forest_build(const Shape& sh, const float* kbar, const float* amax,
                               const float* tau, void* forest, hipStream_t st)
{
    const FsbLayout L = fsb_layout(sh.C, sh.d);
    const int BH = sh.B * sh.H;
    char* F = static_cast<char*>(forest);
    forest_admit_kernel<<<BH, 256, 0, st>>>(amax, tau, sh.H, L, F);
    const int nodes = L.lev_off[L.n_levels];
    if (nodes > 0) {
        const int per = 256 / sh.d;
        forest_mean_kernel<<<dim3((nodes + per - 1) / per, BH), 256, 0, st>>>(kbar, amax, L, F);
        const dim3 g((sh.C + 255) / 256, L.n_levels, BH);
        if (sh.d == 128) forest_radius_kernel<128><<<g, 256, 0, st>>>(kbar, L, F);
        else forest_radius_kernel<64><<<g, 256, 0, st>>>(kbar, L, F);
    }
    return hipGetLastError();
}

hipError_t launch_beam_select(const Shape& sh, const void* q, const void* k,
                              const void* forest0, const void* forest_tau, int beam, double slack,
                              const float* prior_lambda, const float* prior_sigma, int topk,
                              int32_t* idx, float* score, int32_t* effort, hipStream_t st)
{
    if (sh.nq == 0) return hipSuccess;
    const FsbLayout L = fsb_layout(sh.C, sh.d);
    const dim3 grid(sh.nq, sh.B * sh.H);
    const double inv_sqrt_d = 1.0 / std::sqrt((double)sh.d);
    const float scale_log2 = (float)(1.4426950408889634 * inv_sqrt_d);
    char* f0 = static_cast<char*>(const_cast<void*>(forest0));
    char* ft = static_cast<char*>(const_cast<void*>(forest_tau));
#define FS_BEAM_LAUNCH(E, DD, T, RR)                                                      \
    beam_select_kernel<E, DD, RR><<<grid, 64, 0, st>>>(                                     \
        static_cast<const T*>(q), sh.qs[0], sh.qs[1], sh.qs[2], static_cast<const T*>(k),   \
        sh.kvs[0], sh.kvs[1], sh.kvs[2], sh.H, sh.nq, sh.q_pos0, sh.w, sh.s, L, f0, ft, beam, \
        slack, inv_sqrt_d, scale_log2, prior_lambda, prior_sigma, topk, idx, score, effort)
#define FS_BEAM_DISPATCH(RR)                                                              \
    if (sh.bf16 && sh.d == 128) FS_BEAM_LAUNCH(Bf16, 128, uint16_t, RR);                   \
    else if (sh.bf16) FS_BEAM_LAUNCH(Bf16, 64, uint16_t, RR);                              \
    else if (sh.d == 128) FS_BEAM_LAUNCH(F32, 128, float, RR);                             \
    else FS_BEAM_LAUNCH(F32, 64, float, RR)
    if (k) {
        FS_BEAM_DISPATCH(true);
    } else {
        FS_BEAM_DISPATCH(false);
    }
#undef FS_BEAM_DISPATCH
#undef FS_BEAM_LAUNCH
    return hipGetLastError();
}

}  // namespace fs
