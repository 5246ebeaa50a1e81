// Lane helpers of the one-target-per-wave fp32 streaming kernels (attn_f32.hip,
// attn_bwd.hip): lane l holds channels 2l, 2l + 1 (head l / 4) of every
// component; the 4 lanes of a head reduce by two xor shuffles, and each evaluates
// every fourth Gaussian of the distance expansion (FlashSchNet page, section 2.1:
// distance, Gaussian expansion, cosine envelope, computed in the kernel).
#pragma once

#include "e2v2_internal.h"

namespace e2v2 {
namespace lane2 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRsqrt8 = 0.35355339059327373f;
constexpr float kGsc = 0.84932180028801904f;    // sqrt(log2(e) / 2): exp(-t^2 / 2) = exp2(-(kGsc t)^2)

__device__ __forceinline__ float quad_sum(float x)
{
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    return x;
}

// Per-lane share of the distance bias of the lane's head, log2 domain.
struct BiasLane {
    float w[16];        // log2(e) W_rbf[4 kk + r][head], zero past R
    float inv_delta;    // kGsc (R - 1) / cutoff
    float cos_scale;    // 1 / (2 cutoff): cos(pi d / rc) = cos(2 pi * d cos_scale)
    float cutoff;       // the envelope and its slope are 0 from here on (cutoff mask)
    float t_off;        // kGsc * r
    int kk_n;           // ceil(R / 4)

    __device__ __forceinline__ void init(const float *w_rbf, int H, int R, float cutoff, int head, int r)
    {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int k = 4 * kk + r;
            w[kk] = k < R ? w_rbf[k * H + head] * kLog2e : 0.f;
        }
        inv_delta = kGsc * (float)(R - 1) / cutoff;
        cos_scale = 0.5f / cutoff;
        this->cutoff = cutoff;
        t_off = kGsc * (float)r;
        kk_n = (R + 3) >> 2;
    }
    // b_h(d) * log2(e), summed over the head's 4 lanes
    __device__ __forceinline__ float bias2(float d) const
    {
        const float fc = d < cutoff ? 0.5f * (__builtin_amdgcn_cosf(d * cos_scale) + 1.f) : 0.f;
        const float t0 = fmaf(d, inv_delta, -t_off);
        float s = 0.f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            if (kk < kk_n) {
                const float tk = t0 - (4.f * kGsc) * (float)kk;
                s = fmaf(w[kk], __builtin_amdgcn_exp2f(-tk * tk), s);
            }
        return fc * quad_sum(s);
    }
    // The same bias (log2 domain) and its slope db_h/dd in natural units:
    // b = fc S0, db/dd = fc' S0 - fc S1 / (kGsc Delta) with S0 = sum W phi_k,
    // S1 = sum W phi_k t_k, t_k = kGsc (d - mu_k) / Delta (phi_k' = -phi_k (d - mu_k) / Delta^2).
    __device__ __forceinline__ void bias2_slope(float d, float &b2, float &slope) const
    {
        const bool in = d < cutoff;
        const float fc = in ? 0.5f * (__builtin_amdgcn_cosf(d * cos_scale) + 1.f) : 0.f;
        const float fcp = in ? -(0.5f * 3.14159265358979f * 2.f) * cos_scale * __builtin_amdgcn_sinf(d * cos_scale) : 0.f;
        const float t0 = fmaf(d, inv_delta, -t_off);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            if (kk < kk_n) {
                const float tk = t0 - (4.f * kGsc) * (float)kk;
                const float wp = w[kk] * __builtin_amdgcn_exp2f(-tk * tk);
                s0 += wp;
                s1 = fmaf(wp, tk, s1);
            }
        s0 = quad_sum(s0);
        s1 = quad_sum(s1);
        b2 = fc * s0;
        slope = (fcp * s0 - fc * s1 * (inv_delta / (kGsc * kGsc))) * (1.f / kLog2e);
    }
};

// Sum over the wave of each lane's value, taking lanes with `take` only; every
// lane gets the total.
__device__ __forceinline__ float wave_sum_if(float x, bool take)
{
    x = take ? x : 0.f;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// |r_s - r_t| in fp32, one fixed operation order (target t, source s)
__device__ __forceinline__ float pair_dist(const float4 &pt, const float4 &ps)
{
    const float dx = ps.x - pt.x, dy = ps.y - pt.y, dz = ps.z - pt.z;
    return __builtin_amdgcn_sqrtf(fmaf(dz, dz, fmaf(dy, dy, dx * dx)));
}

__device__ __forceinline__ float2 ld2(const float *p) { return *reinterpret_cast<const float2 *>(p); }

// Slot -> node with one contiguous run of slots per XCD (workgroups go to the 8
// XCDs round robin, 4 waves each), then through the optional processing order;
// -1 past the end.
__device__ __forceinline__ int node_of_wave(int n, const int32_t *order)
{
    const int nb = gridDim.x, xcd = blockIdx.x & 7, kth = blockIdx.x >> 3;
    const int lb = xcd * (nb >> 3) + (xcd < (nb & 7) ? xcd : (nb & 7)) + kth;
    const int slot = lb * 4 + (int)(threadIdx.x >> 6);
    if (slot >= n) return -1;
    return order ? order[slot] : slot;
}

}  // namespace lane2
}  // namespace e2v2
