// Target coupling + output projection for 16-bit storage (E2Former-V2 explainer,
// section 3.1: the aggregated message m_i is coupled with the target's own
// encoding, hhat_i = EAAS_i(m_i), then out_i = W_O[l] hhat_i per degree).  m_i
// arrives in fp16 under one power-of-two scale per node.
//
// One block covers 16 nodes and all C channels, in two halves of C/2 input
// channels (one for C = 32): each thread couples 2 channels of one node in
// registers (the node's
// Wigner-D blocks and the path weights staged in LDS), splits hhat into bf16
// hi + lo and writes them to LDS; wave nb then accumulates output channels
// 16 nb .. 16 nb + 15 of every component on v_mfma_f32_16x16x32_bf16 (A = packed
// W_O^T fragment, B = the 16 nodes' hhat rows), hi and lo as two products.  The
// coupling is per channel, so each half of the input channels is complete on
// its own and the contraction is split at the half.
#include "e2v2_internal.h"

namespace e2v2 {

namespace {
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
}  // namespace

template <int L, int C>
__global__ __launch_bounds__(4 * C) __attribute__((amdgpu_waves_per_eu(L <= 2 ? 4 : 1))) void eaas_outproj_kernel(const EaasOutArgs a, const EaasCoef tab)
{
    constexpr int NC = n_comp(L), KB = C / 32, P = path_count(L);
    constexpr int NDM = n_dmat(L);
    constexpr int ND = NDM > 0 ? NDM : 1;
    constexpr int NH = C >= 64 ? 2 : 1;           // input-channel halves (one for C = 32)
    constexpr int CH = C / NH;                    // input channels per half
    constexpr int KBH = KB / NH;                  // 32-channel contraction blocks per half
    constexpr int ROW = NC * CH * 2 + 16;         // LDS bytes per node row of one half (pad spreads banks)
    constexpr int WS = (P & 1) ? P : P + 1;       // LDS stride of one channel's path weights (odd)
    constexpr int NT = 4 * C;
    constexpr int PW = (P * C + NT - 1) / NT;
    constexpr int PD = (16 * ND + NT - 1) / NT;
    constexpr int IPT = 16 * (CH / 2) / NT;       // (node, channel pair) items per thread and half
    __shared__ __align__(16) unsigned char sHi[16 * ROW];
    __shared__ __align__(16) unsigned char sLo[16 * ROW];
    __shared__ float sD[16 * ND];
    __shared__ float sW[C * WS];
    __shared__ float sDir[16];

    const int t = threadIdx.x, lane = t & 63, nb = t >> 6, g = lane >> 4, nl = lane & 15;
    const long long node0 = (long long)blockIdx.x * 16;
    const int nvalid = (a.n - node0) < 16 ? (int)(a.n - node0) : 16;

    // Stage the D blocks, the path weights and the direction flags.
#pragma unroll
    for (int r = 0; r < PW; ++r) {
        const int u = t + r * NT;
        if (u < P * C) {
            const int p = u / C, c = u - p * C;
            sW[c * WS + p] = a.w_tgt[u];
        }
    }
#pragma unroll
    for (int r = 0; r < PD; ++r) {
        const int u = t + r * NT;
        if (u < 16 * ND) sD[u] = (NDM > 0 && u / ND < nvalid) ? a.dmat[node0 * ND + u] : 0.f;
    }
    if (t < 16) {
        float f = 0.f;
        if (t < nvalid) {
            const float4 p4 = a.pos4[node0 + t];
            f = (p4.x != 0.f || p4.y != 0.f || p4.z != 0.f) ? 1.f : 0.f;
        }
        sDir[t] = f;
    }
    __syncthreads();

    // Projection layout: lane (g, nl) accumulates channels 16 nb + 4 g + (0..3) of node nl.
    floatx4 acc[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto afrag = [&](int l, int kb) {
        return __builtin_bit_cast(bf16x8, a.wo[(size_t)l * (C * C / 8) + (nb * KB + kb) * 64 + lane]);
    };

    // Couple every half first (the last half stays in registers), then run one
    // contraction pass per half, so the accumulators are never live during the
    // coupling.  Item t + r NT covers channels 2 cp, 2 cp + 1 of a half, node en.
    auto couple = [&](int half, int r, float (&v)[NC][2]) {
        const int item = t + r * NT;
        const int en = item / (CH / 2), cp = item - en * (CH / 2);
        const long long enode = node0 + en;
        const int c0 = half * CH + 2 * cp;
        const float sc = en < nvalid ? a.msc[enode] : 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            uint32_t x = 0u;
            if (en < nvalid) x = *reinterpret_cast<const uint32_t *>(a.m + (enode * NC + e) * C + c0);
            v[e][0] = (float)__builtin_bit_cast(_Float16, uint16_t(x & 0xffffu)) * sc;
            v[e][1] = (float)__builtin_bit_cast(_Float16, uint16_t(x >> 16)) * sc;
        }
        eaas_multi<L, 2>(v, sD + en * ND, &sW[c0 * WS], WS, tab, sDir[en]);
        if (a.hhat_tap && en < nvalid) {
#pragma unroll
            for (int e = 0; e < NC; ++e)
                *reinterpret_cast<float2 *>(a.hhat_tap + (enode * NC + e) * C + c0) = make_float2(v[e][0], v[e][1]);
        }
    };
    auto stage = [&](int r, const float (&v)[NC][2]) {
        const int item = t + r * NT;
        const int en = item / (CH / 2), cp = item - en * (CH / 2);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            const uint16_t h0 = f_to_bf16(v[e][0]), h1 = f_to_bf16(v[e][1]);
            const uint16_t l0 = f_to_bf16(v[e][0] - bf16_to_f(h0)), l1 = f_to_bf16(v[e][1] - bf16_to_f(h1));
            const int off = en * ROW + (e * CH + 2 * cp) * 2;
            *reinterpret_cast<uint32_t *>(sHi + off) = h0 | (uint32_t(h1) << 16);
            *reinterpret_cast<uint32_t *>(sLo + off) = l0 | (uint32_t(l1) << 16);
        }
    };
    auto contract = [&](int half) {
        const int boff = nl * ROW + g * 16;
#pragma unroll
        for (int l = 0; l <= L; ++l) {
            bf16x8 wf[KBH];
#pragma unroll
            for (int kb = 0; kb < KBH; ++kb) wf[kb] = afrag(l, half * KBH + kb);
#pragma unroll
            for (int m = 0; m < 2 * l + 1; ++m) {
                const int e = l * l + m;
#pragma unroll
                for (int kb = 0; kb < KBH; ++kb) {
                    const int o = boff + e * (CH * 2) + kb * 64;
                    const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sHi + o));
                    const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sLo + o));
                    acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[kb], bh, acc[e], 0, 0, 0);
                    acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[kb], bl, acc[e], 0, 0, 0);
                }
            }
        }
    };
    float vlast[IPT][NC][2];
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
        float v[NC][2];
        couple(0, r, v);
        stage(r, v);
    }
    if constexpr (NH > 1) {
#pragma unroll
        for (int r = 0; r < IPT; ++r) couple(1, r, vlast[r]);
    }
    __syncthreads();
    contract(0);
    if constexpr (NH > 1) {
        __syncthreads();                          // the second half overwrites the tile
#pragma unroll
        for (int r = 0; r < IPT; ++r) stage(r, vlast[r]);
        __syncthreads();
        contract(1);
    }
    if (nl < nvalid) {
        const long long node = node0 + nl;
        if (a.out_bf16) {                        // the next layer's bf16 input, rounded once
#pragma unroll
            for (int e = 0; e < NC; ++e)
                *reinterpret_cast<uint2 *>(a.out_bf16 + (node * NC + e) * C + 16 * nb + 4 * g) =
                    make_uint2(uint32_t(f_to_bf16(acc[e][0])) | (uint32_t(f_to_bf16(acc[e][1])) << 16),
                               uint32_t(f_to_bf16(acc[e][2])) | (uint32_t(f_to_bf16(acc[e][3])) << 16));
        } else {
#pragma unroll
            for (int e = 0; e < NC; ++e)
                *reinterpret_cast<float4 *>(a.out + (node * NC + e) * C + 16 * nb + 4 * g) =
                    make_float4(acc[e][0], acc[e][1], acc[e][2], acc[e][3]);
        }
    }
}

template <int L>
static hipError_t launch_eaas_outproj_l(const EaasOutArgs &a, int C, hipStream_t stream)
{
    const EaasCoef &tab = eaas_table(L);
    const dim3 grid((unsigned)((a.n + 15) / 16));
    switch (C) {
    case 32: eaas_outproj_kernel<L, 32><<<grid, 128, 0, stream>>>(a, tab); break;
    case 64: eaas_outproj_kernel<L, 64><<<grid, 256, 0, stream>>>(a, tab); break;
    case 128: eaas_outproj_kernel<L, 128><<<grid, 512, 0, stream>>>(a, tab); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_eaas_outproj(int L, const EaasOutArgs &a, int C, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    switch (L) {
    case 0: return launch_eaas_outproj_l<0>(a, C, stream);
    case 1: return launch_eaas_outproj_l<1>(a, C, stream);
    case 2: return launch_eaas_outproj_l<2>(a, C, stream);
    case 3: return launch_eaas_outproj_l<3>(a, C, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
