// Gradient of the streaming neighbour attention (fp32 storage).
//
// Forward (E2Former-V2 explainer, section 3.1; distance bias as in the
// FlashSchNet page, section 2.1): s_ij = q_i^h . k_j^h / sqrt(8) + b_h(d_ij),
// alpha_ij = softmax_j(s_ij) per head, m_i = sum_j alpha_ij h'_j.  With
// dm_i = dL/dm_i the gradient is
//   dalpha_ij = <dm_i, h'_j>_h            (sum over the head's channels, all components)
//   dd_i      = sum_j alpha_ij dalpha_ij  (per head)
//   ds_ij     = alpha_ij (dalpha_ij - dd_i)
//   dq_i      = sum_j ds_ij k_j / sqrt(8)        -- target pass, row i
//   dk_j      = sum_i ds_ij q_i / sqrt(8)        -- source pass, row j
//   dh'_j     = sum_i alpha_ij dm_i               -- source pass, row j
// The bias depends on positions only and gets no gradient here.
//
// Target pass: one wave per target streams its row once with an online softmax
// (running maximum M): Z = sum e_j, A = sum e_j dalpha_j, B = sum e_j dalpha_j k_j,
// K = sum e_j k_j with e_j = 2^(s2_j - M), then dd = A / Z and
// dq = (B - dd K) / (Z sqrt(8)).  It stores M and 1 / Z per head.
// Source pass: one wave per source j walks row j of the same list -- for a list
// within a cutoff, i is in row j exactly when j is in row i, so row j names the
// targets that read source j -- recomputes s_ij exactly as the target pass did
// (same operations, same order), alpha_ij = 2^(s2_ij - M_i) / Z_i, and
// accumulates dh'_j and dk_j in registers: every row written by one wave, no
// atomics (FlashSchNet page, section 2.3: owner-computes rows).
//
// Lane layout: lane l holds channels 2l, 2l + 1 (head l / 4) of every component;
// the 4 lanes of a head reduce by two xor shuffles.  With fewer than 16 heads the
// lanes past 4H idle.  Each lane of a head evaluates every fourth Gaussian of the
// distance expansion.
#include "attn_lane2.h"

namespace e2v2 {
using namespace lane2;


template <int L, int H>
__global__ __launch_bounds__(256) void k_attn_bwd_target(const AttnBwdArgs A)
{
    constexpr int NC = n_comp(L), C = 8 * H;
    const int lane = threadIdx.x & 63;
    const int i = __builtin_amdgcn_readfirstlane(node_of_wave(A.n, A.order));
    if (i < 0 || i >= A.n) return;                       // wave-uniform
    const bool act = lane < 4 * H;
    const int c0 = act ? 2 * lane : 0, head = c0 >> 3, r = lane & 3;
    BiasLane bl;
    bl.init(A.w_rbf, A.H, A.R, A.cutoff, head, r);

    const float2 q = ld2(A.q + (size_t)i * C + c0);
    float2 dm[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) dm[e] = ld2(A.dm + ((size_t)i * NC + e) * C + c0);
    const float4 pi4 = A.pos4[i];
    const int start = __builtin_amdgcn_readfirstlane(A.nbr_start[i]);
    const int len = __builtin_amdgcn_readfirstlane(A.nbr_len[i]);

    float M = -INFINITY, Z = 0.f, Aa = 0.f;
    float2 Bk = make_float2(0.f, 0.f), Ck = make_float2(0.f, 0.f);
    for (int p = 0; p < len; ++p) {
        const int j = __builtin_amdgcn_readfirstlane(A.nbr_idx[start + p]);
        if (j < 0 || j >= A.n) continue;                 // wave-uniform
        const float2 kj = ld2(A.k + (size_t)j * C + c0);
        float2 hv[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) hv[e] = ld2(A.hp + ((size_t)j * NC + e) * C + c0);
        const float d = pair_dist(pi4, A.pos4[j]);
        const float qk = quad_sum(fmaf(q.y, kj.y, q.x * kj.x));
        const float s2 = fmaf(qk, kLog2e * kRsqrt8, bl.bias2(d));
        float da = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) da = fmaf(dm[e].y, hv[e].y, fmaf(dm[e].x, hv[e].x, da));
        da = quad_sum(da);
        const float Mn = fmaxf(M, s2);
        const float corr = __builtin_amdgcn_exp2f(M - Mn);
        const float ep = __builtin_amdgcn_exp2f(s2 - Mn);
        const float eda = ep * da;
        Z = fmaf(Z, corr, ep);
        Aa = fmaf(Aa, corr, eda);
        Bk.x = fmaf(Bk.x, corr, eda * kj.x);
        Bk.y = fmaf(Bk.y, corr, eda * kj.y);
        Ck.x = fmaf(Ck.x, corr, ep * kj.x);
        Ck.y = fmaf(Ck.y, corr, ep * kj.y);
        M = Mn;
    }
    float2 dq = make_float2(0.f, 0.f);
    float rz = 0.f, dd = 0.f, mx = INFINITY;             // an empty row: alpha = 0 for every pair
    if (Z > 0.f) {
        rz = 1.f / Z;
        dd = Aa * rz;
        dq.x = (Bk.x - dd * Ck.x) * (rz * kRsqrt8);
        dq.y = (Bk.y - dd * Ck.y) * (rz * kRsqrt8);
        mx = M;
    }
    if (act) {
        *reinterpret_cast<float2 *>(A.dq + (size_t)i * C + c0) = dq;
        if (r == 0) {
            A.mx[(size_t)i * H + head] = mx;
            A.rz[(size_t)i * H + head] = rz;
            A.dd[(size_t)i * H + head] = dd;
        }
    }
}

template <int L, int H>
__global__ __launch_bounds__(256) void k_attn_bwd_source(const AttnBwdArgs A)
{
    constexpr int NC = n_comp(L), C = 8 * H;
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(node_of_wave(A.n, A.order));
    if (j < 0 || j >= A.n) return;                       // wave-uniform
    const bool act = lane < 4 * H;
    const int c0 = act ? 2 * lane : 0, head = c0 >> 3, r = lane & 3;
    BiasLane bl;
    bl.init(A.w_rbf, A.H, A.R, A.cutoff, head, r);

    const float2 kj = ld2(A.k + (size_t)j * C + c0);
    float2 hv[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) hv[e] = ld2(A.hp + ((size_t)j * NC + e) * C + c0);
    const float4 pj4 = A.pos4[j];
    const int start = __builtin_amdgcn_readfirstlane(A.nbr_start[j]);
    const int len = __builtin_amdgcn_readfirstlane(A.nbr_len[j]);

    float2 dh[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) dh[e] = make_float2(0.f, 0.f);
    float2 dk = make_float2(0.f, 0.f);
    for (int p = 0; p < len; ++p) {
        const int i = __builtin_amdgcn_readfirstlane(A.nbr_idx[start + p]);
        if (i < 0 || i >= A.n) continue;                 // wave-uniform
        const float2 qi = ld2(A.q + (size_t)i * C + c0);
        float2 dmi[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) dmi[e] = ld2(A.dm + ((size_t)i * NC + e) * C + c0);
        const float mxi = A.mx[(size_t)i * H + head], rzi = A.rz[(size_t)i * H + head];
        const float ddi = A.dd[(size_t)i * H + head];
        const float d = pair_dist(A.pos4[i], pj4);
        const float qk = quad_sum(fmaf(qi.y, kj.y, qi.x * kj.x));
        const float s2 = fmaf(qk, kLog2e * kRsqrt8, bl.bias2(d));
        const float al = __builtin_amdgcn_exp2f(s2 - mxi) * rzi;
        float da = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) da = fmaf(dmi[e].y, hv[e].y, fmaf(dmi[e].x, hv[e].x, da));
        da = quad_sum(da);
        const float ds = al * (da - ddi);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            dh[e].x = fmaf(al, dmi[e].x, dh[e].x);
            dh[e].y = fmaf(al, dmi[e].y, dh[e].y);
        }
        dk.x = fmaf(ds, qi.x, dk.x);
        dk.y = fmaf(ds, qi.y, dk.y);
    }
    if (act) {
#pragma unroll
        for (int e = 0; e < NC; ++e) *reinterpret_cast<float2 *>(A.dhp + ((size_t)j * NC + e) * C + c0) = dh[e];
        *reinterpret_cast<float2 *>(A.dk + (size_t)j * C + c0) = make_float2(dk.x * kRsqrt8, dk.y * kRsqrt8);
    }
}

template <int L, int H>
static hipError_t launch_bwd_lh(const AttnBwdArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.n + 3) / 4));
    k_attn_bwd_target<L, H><<<grid, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_attn_bwd_source<L, H><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
}

template <int L>
static hipError_t launch_bwd_l(const AttnBwdArgs &a, hipStream_t stream)
{
    switch (a.H) {
    case 4: return launch_bwd_lh<L, 4>(a, stream);
    case 8: return launch_bwd_lh<L, 8>(a, stream);
    case 16: return launch_bwd_lh<L, 16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_bwd(int L, const AttnBwdArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    if (a.C != 8 * a.H || a.R < 2 || a.R > 64) return hipErrorInvalidValue;
    switch (L) {
    case 0: return launch_bwd_l<0>(a, stream);
    case 1: return launch_bwd_l<1>(a, stream);
    case 2: return launch_bwd_l<2>(a, stream);
    case 3: return launch_bwd_l<3>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
