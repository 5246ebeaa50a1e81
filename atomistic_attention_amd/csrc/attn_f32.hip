// Streaming neighbour attention for fp32 storage, with the target coupling in
// its epilogue.
//
// E2Former-V2 explainer, section 3.1 (the message m_i = sum_j alpha_ij h'_j
// formed on the fly, then coupled with the target's own encoding) and section
// 3.2 (online softmax with a running maximum and normaliser, each key and value
// row read once per target, accumulation on chip, padded entries skipped); the
// distance bias is computed in the kernel (FlashSchNet page, section 2.1).
//
// One 64-lane wave per target: lane l holds channels 2l, 2l + 1 of every
// component (lanes past 4H idle), so a neighbour's key row and each component of
// its value row arrive as one 8-byte load per lane, 512 contiguous bytes per
// wave.  Per pair: the 4 lanes of a head finish q . k with two shuffles, add the
// log2-domain bias, and fold the pair into the running maximum, normaliser and
// 2 NC accumulators.  The next pair's rows are requested before the current
// pair is folded in.  At the end each lane couples its two channels of m_i with
// the target's D blocks and path weights (EAAS, section 2.1) and writes them.
#include "attn_lane2.h"

namespace e2v2 {
using namespace lane2;

template <int NC>
struct PairRows {
    float2 k, h[NC];
    float4 p;
    int j;
};

template <int L, int H>
__global__ __launch_bounds__(256) void k_attn_f32(const AttnArgs A, const EaasCoef tab)
{
    constexpr int NC = n_comp(L), C = 8 * H, ND = n_dmat(L), P = path_count(L);
    const int lane = threadIdx.x & 63;
    const int i = __builtin_amdgcn_readfirstlane(node_of_wave(A.n, A.order));
    if (i < 0 || i >= A.n) return;                       // wave-uniform
    const bool act = lane < 4 * H;
    const int c0 = act ? 2 * lane : 0, head = c0 >> 3, r = lane & 3;
    BiasLane bl;
    bl.init(A.w_rbf, H, A.R, A.cutoff, head, r);
    const float *K = reinterpret_cast<const float *>(A.k);
    const float *HP = reinterpret_cast<const float *>(A.hp);

    const float2 q = ld2(A.q + (size_t)i * C + c0);
    const float4 pi4 = A.pos4[i];
    const int start = __builtin_amdgcn_readfirstlane(A.nbr_start[i]);
    const int len = __builtin_amdgcn_readfirstlane(A.nbr_len[i]);
    auto fetch = [&](int p, PairRows<NC> &x) {
        int j = p < len ? __builtin_amdgcn_readfirstlane(A.nbr_idx[start + p]) : -1;
        if (j >= A.n) j = -1;
        x.j = j;
        const size_t node = (size_t)(j >= 0 ? j : i);   // an in-bounds row for skipped entries
        x.k = ld2(K + node * C + c0);
#pragma unroll
        for (int e = 0; e < NC; ++e) x.h[e] = ld2(HP + (node * NC + e) * C + c0);
        x.p = A.pos4[node];
    };

    float M = -INFINITY, Z = 0.f;
    float2 acc[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) acc[e] = make_float2(0.f, 0.f);
    PairRows<NC> cur, nxt;
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
            for (int e = 0; e < NC; ++e) {
                acc[e].x = fmaf(acc[e].x, corr, ep * cur.h[e].x);
                acc[e].y = fmaf(acc[e].y, corr, ep * cur.h[e].y);
            }
            M = Mn;
        }
        cur = nxt;
    }
    const float rz = Z > 0.f ? 1.f / Z : 0.f;            // an empty row gives m_i = 0
    float m0[NC], m1[NC], y0[NC], y1[NC], w0[P], w1[P];
#pragma unroll
    for (int e = 0; e < NC; ++e) {
        m0[e] = acc[e].x * rz;
        m1[e] = acc[e].y * rz;
    }
    if (!act) return;
    if (A.m_tap) {
#pragma unroll
        for (int e = 0; e < NC; ++e)
            *reinterpret_cast<float2 *>(A.m_tap + ((size_t)i * NC + e) * C + c0) = make_float2(m0[e], m1[e]);
    }
    // target coupling with the target's own frame (zero position: l_f > 0 paths vanish)
    const float *Di = A.dmat + (size_t)i * (ND > 0 ? ND : 1);
    const bool dir = (pi4.x != 0.f) || (pi4.y != 0.f) || (pi4.z != 0.f);
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const float2 wv = ld2(A.w_tgt + p * C + c0);
        w0[p] = wv.x;
        w1[p] = wv.y;
    }
    eaas_channel<L>(Di, m0, y0, w0, tab, dir);
    eaas_channel<L>(Di, m1, y1, w1, tab, dir);
#pragma unroll
    for (int e = 0; e < NC; ++e)
        *reinterpret_cast<float2 *>(A.hhat + ((size_t)i * NC + e) * C + c0) = make_float2(y0[e], y1[e]);
}

template <int L>
static hipError_t launch_f32_l(const AttnArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.n + 3) / 4)), block(256);
    const EaasCoef &tab = eaas_table(L);
    switch (a.H) {
    case 4: k_attn_f32<L, 4><<<grid, block, 0, stream>>>(a, tab); break;
    case 8: k_attn_f32<L, 8><<<grid, block, 0, stream>>>(a, tab); break;
    case 16: k_attn_f32<L, 16><<<grid, block, 0, stream>>>(a, tab); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_f32(int L, const AttnArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    if (a.C != 8 * a.H || a.R < 2 || a.R > 64) return hipErrorInvalidValue;
    switch (L) {
    case 0: return launch_f32_l<0>(a, stream);
    case 1: return launch_f32_l<1>(a, stream);
    case 2: return launch_f32_l<2>(a, stream);
    case 3: return launch_f32_l<3>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
