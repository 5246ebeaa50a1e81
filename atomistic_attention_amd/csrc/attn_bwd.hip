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
// Source pass: one wave per source j walks row j of the transposed list (the
// targets that read source j; for a symmetric list, the list itself), recomputes
// s_ij exactly as the target pass did
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


template <int L, int H, bool POS>
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
    // POS: the bias-slope sums U = sum e dalpha b' u, V = sum e b' u (u = (r_i - r_j) / d)
    // and the message m_i itself
    float3 Uf = make_float3(0.f, 0.f, 0.f), Vf = make_float3(0.f, 0.f, 0.f);
    float2 am[POS ? NC : 1];
#pragma unroll
    for (int e = 0; e < (POS ? NC : 1); ++e) am[e] = make_float2(0.f, 0.f);
    for (int p = 0; p < len; ++p) {
        const int j = __builtin_amdgcn_readfirstlane(A.nbr_idx[start + p]);
        if (j < 0 || j >= A.n) continue;                 // wave-uniform
        const float2 kj = ld2(A.k + (size_t)j * C + c0);
        float2 hv[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) hv[e] = ld2(A.hp + ((size_t)j * NC + e) * C + c0);
        const float4 pj4 = A.pos4[j];
        const float d = pair_dist(pi4, pj4);
        float b2, slope = 0.f;
        if constexpr (POS) bl.bias2_slope(d, b2, slope);
        else b2 = bl.bias2(d);
        const float qk = quad_sum(fmaf(q.y, kj.y, q.x * kj.x));
        const float s2 = fmaf(qk, kLog2e * kRsqrt8, b2);
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
        if constexpr (POS) {
            const float id = d > 0.f ? 1.f / d : 0.f;    // coincident atoms: no direction, no term
            const float ux = (pi4.x - pj4.x) * id, uy = (pi4.y - pj4.y) * id, uz = (pi4.z - pj4.z) * id;
            const float eb = ep * slope, ebd = eb * da;
            Uf.x = fmaf(Uf.x, corr, ebd * ux);
            Uf.y = fmaf(Uf.y, corr, ebd * uy);
            Uf.z = fmaf(Uf.z, corr, ebd * uz);
            Vf.x = fmaf(Vf.x, corr, eb * ux);
            Vf.y = fmaf(Vf.y, corr, eb * uy);
            Vf.z = fmaf(Vf.z, corr, eb * uz);
#pragma unroll
            for (int e = 0; e < (POS ? NC : 1); ++e) {
                am[e].x = fmaf(am[e].x, corr, ep * hv[e].x);
                am[e].y = fmaf(am[e].y, corr, ep * hv[e].y);
            }
        }
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
    if constexpr (POS) {
        // dL/dr_i from the pairs (i, j): sum over heads of (U - dd V) / Z; the 4
        // lanes of a head hold the same values, so one lane per head contributes
        const bool take = act && r == 0;
        const float fx = wave_sum_if((Uf.x - dd * Vf.x) * rz, take);
        const float fy = wave_sum_if((Uf.y - dd * Vf.y) * rz, take);
        const float fz = wave_sum_if((Uf.z - dd * Vf.z) * rz, take);
        if (lane == 0) {
            float *gpi = A.grad_pos + 3 * (size_t)i;
            gpi[0] = A.pos_acc ? gpi[0] + fx : fx;
            gpi[1] = A.pos_acc ? gpi[1] + fy : fy;
            gpi[2] = A.pos_acc ? gpi[2] + fz : fz;
        }
        if (act) {
#pragma unroll
            for (int e = 0; e < (POS ? NC : 1); ++e)
                *reinterpret_cast<float2 *>(A.m + ((size_t)i * NC + e) * C + c0) = make_float2(am[e].x * rz, am[e].y * rz);
        }
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

template <int L, int H, bool POS>
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
    const int start = __builtin_amdgcn_readfirstlane(A.src_start[j]);
    const int len = __builtin_amdgcn_readfirstlane(A.src_len[j]);

    float2 dh[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) dh[e] = make_float2(0.f, 0.f);
    float2 dk = make_float2(0.f, 0.f);
    float3 Fj = make_float3(0.f, 0.f, 0.f);              // POS: sum_i ds_ij b'(d_ij) (r_j - r_i) / d_ij
    for (int p = 0; p < len; ++p) {
        const int i = __builtin_amdgcn_readfirstlane(A.src_idx[start + p]);
        if (i < 0 || i >= A.n) continue;                 // wave-uniform
        const float2 qi = ld2(A.q + (size_t)i * C + c0);
        float2 dmi[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) dmi[e] = ld2(A.dm + ((size_t)i * NC + e) * C + c0);
        const float mxi = A.mx[(size_t)i * H + head], rzi = A.rz[(size_t)i * H + head];
        const float ddi = A.dd[(size_t)i * H + head];
        const float4 pi4 = A.pos4[i];
        const float d = pair_dist(pi4, pj4);
        float b2, slope = 0.f;
        if constexpr (POS) bl.bias2_slope(d, b2, slope);
        else b2 = bl.bias2(d);
        const float qk = quad_sum(fmaf(qi.y, kj.y, qi.x * kj.x));
        const float s2 = fmaf(qk, kLog2e * kRsqrt8, b2);
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
        if constexpr (POS) {
            const float id = d > 0.f ? 1.f / d : 0.f;
            const float sb = ds * slope * id;
            Fj.x = fmaf(sb, pj4.x - pi4.x, Fj.x);
            Fj.y = fmaf(sb, pj4.y - pi4.y, Fj.y);
            Fj.z = fmaf(sb, pj4.z - pi4.z, Fj.z);
        }
    }
    if constexpr (POS) {                                 // after the target pass wrote row j
        const bool take = act && r == 0;
        const float fx = wave_sum_if(Fj.x, take), fy = wave_sum_if(Fj.y, take), fz = wave_sum_if(Fj.z, take);
        if (lane == 0) {
            A.grad_pos[3 * (size_t)j + 0] += fx;
            A.grad_pos[3 * (size_t)j + 1] += fy;
            A.grad_pos[3 * (size_t)j + 2] += fz;
        }
    }
    if (act) {
#pragma unroll
        for (int e = 0; e < NC; ++e) *reinterpret_cast<float2 *>(A.dhp + ((size_t)j * NC + e) * C + c0) = dh[e];
        *reinterpret_cast<float2 *>(A.dk + (size_t)j * C + c0) = make_float2(dk.x * kRsqrt8, dk.y * kRsqrt8);
    }
}

// ---------------------------------------------------------------------------
// Encoding term of dL/dpos.  The couplings read node i's own encoding Y(r_i / |r_i|)
// (explainer section 2.1; the EAAS form equals the dense tensor product,
// Proposition 4.3), so dL/dY_i[ef] = sum_c sum over the entries T_p[e_i, ef, e_o] of
// w_p[c] x[e_i][c] g[e_o][c] for (x, g, w) = (v, dh', w_src) and (m, dhhat, w_tgt).
// Then dL/dr = (I - u u^T) grad P(u) / |r|, u = r / |r|, for the polynomial forms P
// of the real harmonics (any extension off the sphere gives the same tangent part).
// The entries are those of ygrad_terms (the selection rules of the real basis).

// grad P of each harmonic component ef = 1 .. (L+1)^2 - 1 at (x, y, z), into G[ef - 1]
template <int L>
__device__ __forceinline__ void sh_poly_grad(float x, float y, float z, float (*G)[3])
{
    const float s3 = 1.7320508075688772f;
    G[0][0] = 0.f; G[0][1] = s3; G[0][2] = 0.f;                  // sqrt3 y
    G[1][0] = 0.f; G[1][1] = 0.f; G[1][2] = s3;                  // sqrt3 z
    G[2][0] = s3; G[2][1] = 0.f; G[2][2] = 0.f;                  // sqrt3 x
    if constexpr (L >= 2) {
        const float s15 = 3.872983346207417f, s5 = 2.23606797749979f;
        G[3][0] = s15 * y; G[3][1] = s15 * x; G[3][2] = 0.f;     // s15 x y
        G[4][0] = 0.f; G[4][1] = s15 * z; G[4][2] = s15 * y;     // s15 y z
        G[5][0] = 0.f; G[5][1] = 0.f; G[5][2] = 3.f * s5 * z;   // s5 (3 z^2 - 1) / 2
        G[6][0] = s15 * z; G[6][1] = 0.f; G[6][2] = s15 * x;     // s15 x z
        G[7][0] = s15 * x; G[7][1] = -s15 * y; G[7][2] = 0.f;    // s15 (x^2 - y^2) / 2
    }
    if constexpr (L >= 3) {
        const float a = 2.091650066335189f, b = 10.246950765959598f, c = 1.620185174601965f;
        const float d = 1.3228756555322954f;
        G[8][0] = 6.f * a * x * y; G[8][1] = 3.f * a * (x * x - y * y); G[8][2] = 0.f;   // a y (3x^2 - y^2)
        G[9][0] = b * y * z; G[9][1] = b * x * z; G[9][2] = b * x * y;                  // b x y z
        G[10][0] = 0.f; G[10][1] = c * (5.f * z * z - 1.f); G[10][2] = 10.f * c * y * z; // c y (5z^2 - 1)
        G[11][0] = 0.f; G[11][1] = 0.f; G[11][2] = d * (15.f * z * z - 3.f);             // d (5z^3 - 3z)
        G[12][0] = c * (5.f * z * z - 1.f); G[12][1] = 0.f; G[12][2] = 10.f * c * x * z; // c x (5z^2 - 1)
        G[13][0] = b * x * z; G[13][1] = -b * y * z; G[13][2] = 0.5f * b * (x * x - y * y); // b z (x^2 - y^2) / 2
        G[14][0] = 3.f * a * (x * x - y * y); G[14][1] = -6.f * a * x * y; G[14][2] = 0.f; // a x (x^2 - 3y^2)
    }
}

// One wave per node, lanes as in the attention passes (2 channels each): the
// node's four feature rows and both path-weight rows sit in registers, and the
// contraction over the coupling entries is unrolled at compile time.
template <int L, int H>
__global__ __launch_bounds__(256) void k_pos_grad(const PosGradArgs A)
{
    constexpr int NC = n_comp(L), C = 8 * H, P = path_count(L);
    constexpr YTerms T = ygrad_terms<L>();
    const int lane = threadIdx.x & 63;
    const int i = __builtin_amdgcn_readfirstlane(node_of_wave(A.n, nullptr));
    if (i < 0) return;
    const bool act = lane < 4 * H;
    const int c0 = act ? 2 * lane : 0;
    float2 xs[NC], gs[NC], xt[NC], gt[NC], ws[P], wt[P];
#pragma unroll
    for (int e = 0; e < NC; ++e) {
        const size_t o = ((size_t)i * NC + e) * C + c0;
        xs[e] = ld2(A.v + o);
        gs[e] = ld2(A.dhp + o);
        xt[e] = ld2(A.m + o);
        gt[e] = ld2(A.dhhat + o);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        ws[p] = ld2(A.w_src + p * C + c0);
        wt[p] = ld2(A.w_tgt + p * C + c0);
    }
    float acc[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int q = 0; q < T.n; ++q) {
        const YTerm t = T.t[q];
        float s = ws[t.p].x * xs[t.ei].x * gs[t.eo].x;
        s = fmaf(ws[t.p].y * xs[t.ei].y, gs[t.eo].y, s);
        s = fmaf(wt[t.p].x * xt[t.ei].x, gt[t.eo].x, s);
        s = fmaf(wt[t.p].y * xt[t.ei].y, gt[t.eo].y, s);
        acc[t.ef] = fmaf(A.tval[q], s, acc[t.ef]);
    }
    float gy[NC];
#pragma unroll
    for (int ef = 1; ef < NC; ++ef) gy[ef] = wave_sum_if(acc[ef], act);
    if (lane != 0) return;
    const float rx = A.pos[3 * (size_t)i], ry = A.pos[3 * (size_t)i + 1], rz = A.pos[3 * (size_t)i + 2];
    const float nrm = sqrtf(fmaf(rz, rz, fmaf(ry, ry, rx * rx)));
    if (!(nrm > 0.f)) return;               // no direction at the origin: the encoding is held constant
    const float inv = 1.f / nrm, ux = rx * inv, uy = ry * inv, uz = rz * inv;
    float G[NC - 1][3];
    sh_poly_grad<L>(ux, uy, uz, G);
    float gx = 0.f, gyy = 0.f, gz = 0.f;
#pragma unroll
    for (int ef = 1; ef < NC; ++ef) {
        gx = fmaf(gy[ef], G[ef - 1][0], gx);
        gyy = fmaf(gy[ef], G[ef - 1][1], gyy);
        gz = fmaf(gy[ef], G[ef - 1][2], gz);
    }
    const float ug = ux * gx + uy * gyy + uz * gz;
    A.grad_pos[3 * (size_t)i + 0] += (gx - ug * ux) * inv;
    A.grad_pos[3 * (size_t)i + 1] += (gyy - ug * uy) * inv;
    A.grad_pos[3 * (size_t)i + 2] += (gz - ug * uz) * inv;
}

template <int L>
static hipError_t launch_pos_grad_l(const PosGradArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.n + 3) / 4));
    switch (a.H) {
    case 4: k_pos_grad<L, 4><<<grid, 256, 0, stream>>>(a); break;
    case 8: k_pos_grad<L, 8><<<grid, 256, 0, stream>>>(a); break;
    case 16: k_pos_grad<L, 16><<<grid, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pos_grad(int L, const PosGradArgs &a, hipStream_t stream)
{
    if (a.n <= 0 || L == 0) return hipSuccess;           // l_max = 0: the encoding is the constant Y_0
    switch (L) {
    case 1: return launch_pos_grad_l<1>(a, stream);
    case 2: return launch_pos_grad_l<2>(a, stream);
    case 3: return launch_pos_grad_l<3>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int L, int H>
static hipError_t launch_bwd_lh(const AttnBwdArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.n + 3) / 4));
    if (a.grad_pos) k_attn_bwd_target<L, H, true><<<grid, 256, 0, stream>>>(a);
    else k_attn_bwd_target<L, H, false><<<grid, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.grad_pos) k_attn_bwd_source<L, H, true><<<grid, 256, 0, stream>>>(a);
    else k_attn_bwd_source<L, H, false><<<grid, 256, 0, stream>>>(a);
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
