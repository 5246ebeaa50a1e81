// The exact edge-equivalent form, evaluated node by node (E2Former-V2 explainer,
// section 1.2: the Wigner-6j recoupling identity behind node-centric attention).
//
// The edge form couples every neighbour's value with the solid harmonics of the
// edge vector, S(x_ij), x_ij = (r_j - r_i) / r_c.  With an origin o (the centroid
// of the positions) x_ij = x_j + y_i, x_j = (r_j - o) / r_c,
// y_i = (o - r_i) / r_c, and edge_terms.h splits the product into
//   * a source part per node, G_j = blocks (v_j^li (x) S^lam(x_j))^lp
//     (k_edge_source, one thread per node and channel);
//   * the stream, M_i = sum_j alpha_ij G_j with the layer's attention weights
//     (k_edge_attn: one wave per target and group of 20 components, online
//     softmax as in the layer's streaming kernels, no N x K tensor);
//   * a target part, m_i = sum over paths, lam and lp of w_e a U (M_i (x) S^mu(y_i))
//     (k_edge_target, one thread per target and channel).
// The result does not depend on o; o only keeps |x_j| and |y_i| small, since the
// node terms grow like (|r - o| / r_c)^l_f and cancel to the edge term.
#include "attn_lane2.h"
#include "edge_terms.h"

namespace e2v2 {
using namespace lane2;

namespace {

constexpr int kGroup = 20;                // components of G per streaming wave

template <int L>
constexpr int padded_comps()
{
    return (edge::blocks<L>().ncomp + kGroup - 1) / kGroup * kGroup;
}

// Component-normalised real solid harmonics S^l(x) = |x|^l Y^l(x / |x|), l <= L,
// as polynomials; S^0 = 1.
template <int L>
__device__ __forceinline__ void solid(float x, float y, float z, float *S)
{
    S[0] = 1.f;
    if constexpr (L >= 1) {
        const float s3 = 1.7320508075688772f;
        S[1] = s3 * y;
        S[2] = s3 * z;
        S[3] = s3 * x;
    }
    if constexpr (L >= 2) {
        const float s15 = 3.872983346207417f, s5h = 1.118033988749895f;   // sqrt(15), sqrt(5) / 2
        S[4] = s15 * x * y;
        S[5] = s15 * y * z;
        S[6] = s5h * (2.f * z * z - x * x - y * y);
        S[7] = s15 * x * z;
        S[8] = 0.5f * s15 * (x - y) * (x + y);
    }
}

// Centroid of the finite positions, summed in fp64 in a fixed order (one block:
// thread t takes atoms t, t + 1024, ...; then a fixed tree), so the result is the
// same on every call; no finite position gives 0.  The centroid keeps |r - o| small
// for the bulk of the atoms even when a few lie far away.
__global__ __launch_bounds__(1024) void k_edge_origin(const float *__restrict__ pos, int n, float4 *origin)
{
    __shared__ double ss[4][1024];
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (long long i = threadIdx.x; i < n; i += blockDim.x) {
        const float x = pos[3 * i], y = pos[3 * i + 1], z = pos[3 * i + 2];
        if (__builtin_isfinite(x) && __builtin_isfinite(y) && __builtin_isfinite(z)) {
            acc[0] += x;
            acc[1] += y;
            acc[2] += z;
            acc[3] += 1.0;
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) ss[a][threadIdx.x] = acc[a];
    __syncthreads();
    for (int s = 512; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s)
#pragma unroll
            for (int a = 0; a < 4; ++a) ss[a][threadIdx.x] += ss[a][threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double cnt = ss[3][0];
        *origin = cnt > 0.0 ? make_float4((float)(ss[0][0] / cnt), (float)(ss[1][0] / cnt), (float)(ss[2][0] / cnt), 0.f)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// G_j = (v_j^li (x) S^lam(x_j))^lp for every block; the padding past the blocks'
// components is written with zeros.  Also pos4[j] = (r_j, 0).
template <int L>
__global__ __launch_bounds__(256) void k_edge_source(const EdgeArgs A)
{
    constexpr int NC = n_comp(L);
    constexpr edge::SrcTerms T = edge::src_terms<L>();
    constexpr int NG = edge::blocks<L>().ncomp, NGP = padded_comps<L>();
    const int C = A.C;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long long)A.n * C) return;
    const long long j = t / C;
    const int c = (int)(t - j * C);
    const float4 o = *A.origin;
    const float px = A.pos[3 * j], py = A.pos[3 * j + 1], pz = A.pos[3 * j + 2];
    if (c == 0) A.pos4[j] = make_float4(px, py, pz, 0.f);
    const float ir = 1.f / A.cutoff;
    float S[NC], v[NC], g[NG];
    solid<L>((px - o.x) * ir, (py - o.y) * ir, (pz - o.z) * ir, S);
#pragma unroll
    for (int e = 0; e < NC; ++e) v[e] = A.v[(j * NC + e) * C + c];
#pragma unroll
    for (int e = 0; e < NG; ++e) g[e] = 0.f;
#pragma unroll
    for (int q = 0; q < T.n; ++q) g[T.t[q].eg] = fmaf(A.src_val[q] * v[T.t[q].ei], S[T.t[q].el], g[T.t[q].eg]);
    float *out = A.G + j * NGP * C + c;
#pragma unroll
    for (int e = 0; e < NGP; ++e) out[(long long)e * C] = e < NG ? g[e] : 0.f;
}

template <int NW>
struct EdgeRows {
    float2 k, g[NW];
    float4 p;
    int j;
};

// M_i, components [grp * kGroup, (grp + 1) * kGroup) of the padded layout: one wave
// per (target, group), lane l holds channels 2l, 2l + 1 (lanes past 4H idle); the
// logits, distance bias and online softmax are those of the fp32 streaming kernel.
template <int L, int H>
__global__ __launch_bounds__(256) void k_edge_attn(const EdgeArgs A)
{
    constexpr int C = 8 * H, NGP = padded_comps<L>(), NGRP = NGP / kGroup;
    const int lane = threadIdx.x & 63;
    // XCD-aware: each of the 8 XCDs walks one contiguous run of (target, group) slots
    const int nb = gridDim.x, xcd = blockIdx.x & 7, kth = blockIdx.x >> 3;
    const int lb = xcd * (nb >> 3) + (xcd < (nb & 7) ? xcd : (nb & 7)) + kth;
    const long long slot = (long long)lb * 4 + (threadIdx.x >> 6);
    if (slot >= (long long)A.n * NGRP) return;
    const int ts = (int)(slot / NGRP), grp = (int)(slot - (long long)ts * NGRP);
    const int i = __builtin_amdgcn_readfirstlane(A.order ? A.order[ts] : ts);
    if (i < 0 || i >= A.n) return;                       // wave-uniform
    const bool act = lane < 4 * H;
    const int c0 = act ? 2 * lane : 0, head = c0 >> 3, r = lane & 3;
    BiasLane bl;
    bl.init(A.w_rbf, H, A.R, A.cutoff, head, r);
    const float2 q = ld2(A.q + (size_t)i * C + c0);
    const float4 pi4 = A.pos4[i];
    const int start = __builtin_amdgcn_readfirstlane(A.nbr_start[i]);
    const int len = __builtin_amdgcn_readfirstlane(A.nbr_len[i]);
    const float *Gb = A.G + (size_t)grp * kGroup * C + c0;
    auto fetch = [&](int p, EdgeRows<kGroup> &x) {
        int j = p < len ? __builtin_amdgcn_readfirstlane(A.nbr_idx[start + p]) : -1;
        if (j >= A.n) j = -1;
        x.j = j;
        const size_t node = (size_t)(j >= 0 ? j : i);   // an in-bounds row for skipped entries
        x.k = ld2(A.k + node * C + c0);
#pragma unroll
        for (int e = 0; e < kGroup; ++e) x.g[e] = ld2(Gb + (node * NGP + e) * C);
        x.p = A.pos4[node];
    };
    float M = -INFINITY, Z = 0.f;
    float2 acc[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = make_float2(0.f, 0.f);
    EdgeRows<kGroup> cur, nxt;
    fetch(0, cur);
    for (int p = 0; p < len; ++p) {
        fetch(p + 1, nxt);
        if (cur.j >= 0) {                                // wave-uniform
            const float d = pair_dist(pi4, cur.p);
            const float qk = quad_sum(fmaf(q.y, cur.k.y, q.x * cur.k.x));
            const float s2 = fmaf(qk, kLog2e * kRsqrt8, bl.bias2(d));
            const float Mn = fmaxf(M, s2);
            const float corr = __builtin_amdgcn_exp2f(M - Mn);
            const float ep = __builtin_amdgcn_exp2f(s2 - Mn);
            Z = fmaf(Z, corr, ep);
#pragma unroll
            for (int e = 0; e < kGroup; ++e) {
                acc[e].x = fmaf(acc[e].x, corr, ep * cur.g[e].x);
                acc[e].y = fmaf(acc[e].y, corr, ep * cur.g[e].y);
            }
            M = Mn;
        }
        cur = nxt;
    }
    if (!act) return;
    const float rz = Z > 0.f ? 1.f / Z : 0.f;            // an empty row gives M_i = 0
    float *out = A.M + ((size_t)i * NGP + (size_t)grp * kGroup) * C + c0;
#pragma unroll
    for (int e = 0; e < kGroup; ++e)
        *reinterpret_cast<float2 *>(out + (size_t)e * C) = make_float2(acc[e].x * rz, acc[e].y * rz);
}

// m_i = sum over the target terms of w_e[p] val M_i[eg] S(y_i)[em].
template <int L>
__global__ __launch_bounds__(256) void k_edge_target(const EdgeArgs A)
{
    constexpr int NC = n_comp(L), P = path_count(L);
    constexpr edge::TgtTerms T = edge::tgt_terms<L>();
    constexpr int NG = edge::blocks<L>().ncomp, NGP = padded_comps<L>();
    const int C = A.C;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long long)A.n * C) return;
    const long long i = t / C;
    const int c = (int)(t - i * C);
    const float4 o = *A.origin;
    const float ir = 1.f / A.cutoff;
    float S[NC], m[NG], w[P], y[NC];
    solid<L>((o.x - A.pos[3 * i]) * ir, (o.y - A.pos[3 * i + 1]) * ir, (o.z - A.pos[3 * i + 2]) * ir, S);
    const float *Mi = A.M + i * NGP * C + c;
#pragma unroll
    for (int e = 0; e < NG; ++e) m[e] = Mi[(long long)e * C];
#pragma unroll
    for (int p = 0; p < P; ++p) w[p] = A.w_e[p * C + c];
#pragma unroll
    for (int e = 0; e < NC; ++e) y[e] = 0.f;
#pragma unroll
    for (int q = 0; q < T.n; ++q)
        y[T.t[q].eo] = fmaf(w[T.t[q].p] * A.tgt_val[q], m[T.t[q].eg] * S[T.t[q].em], y[T.t[q].eo]);
#pragma unroll
    for (int e = 0; e < NC; ++e) A.medge[(i * NC + e) * C + c] = y[e];
}

template <int L>
hipError_t launch_edge_l(const EdgeArgs &a, hipStream_t stream)
{
    const long long nt = (long long)a.n * a.C;
    const dim3 blk(256), gnc((unsigned)((nt + 255) / 256));
    k_edge_source<L><<<gnc, blk, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int NGRP = padded_comps<L>() / kGroup;
    const dim3 gw((unsigned)(((long long)a.n * NGRP + 3) / 4));
    switch (a.H) {
    case 4: k_edge_attn<L, 4><<<gw, blk, 0, stream>>>(a); break;
    case 8: k_edge_attn<L, 8><<<gw, blk, 0, stream>>>(a); break;
    case 16: k_edge_attn<L, 16><<<gw, blk, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_edge_target<L><<<gnc, blk, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

int edge_padded_comps(int L)
{
    switch (L) {
    case 0: return padded_comps<0>();
    case 1: return padded_comps<1>();
    case 2: return padded_comps<2>();
    default: return -1;
    }
}

hipError_t launch_edge(int L, const EdgeArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    if (a.C != 8 * a.H || a.R < 2 || a.R > 64) return hipErrorInvalidValue;
    k_edge_origin<<<1, 1024, 0, stream>>>(a.pos, a.n, a.origin);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (L) {
    case 0: return launch_edge_l<0>(a, stream);
    case 1: return launch_edge_l<1>(a, stream);
    case 2: return launch_edge_l<2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
