// Helpers shared by the streaming attention kernels (attn.hip, attn_pair.hip):
// the per-lane value-row pieces and small lane utilities.
#pragma once

#include "e2v2_internal.h"

namespace e2v2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// One neighbour's value pieces for this lane's 4 channels.  fp32 h' is
// [node][comp][C]: one 16-byte load per component.  16-bit h' is stored with
// components interleaved in pairs (hp_f16_offset): one 16-byte load covers 4
// channels of two components -- half the load instructions of a per-component
// layout -- and an odd last component travels with the key (hp_pair_row).
template <bool HB, int NC> struct HpStep;
template <int NC> struct HpStep<true, NC> {
    static constexpr int NPR = NC / 2;
    uint4 pr[NPR > 0 ? NPR : 1];
    __device__ __forceinline__ void load(const void *base, int node, int cb, int C)
    {
        const uint16_t *nb = reinterpret_cast<const uint16_t *>(base) + (size_t)node * hp_pair_row(NC, C);
#pragma unroll
        for (int p = 0; p < NPR; ++p) pr[p] = *reinterpret_cast<const uint4 *>(nb + p * 2 * C + (cb >> 2) * 8);
    }
    // component e < 2 NPR, channel c of the lane's 4 (the odd last component
    // comes with the key, see tail())
    __device__ __forceinline__ float get(int e, int c) const
    {
        const uint4 &v = pr[e >> 1];
        const int k = (e & 1) * 2 + (c >> 1);
        const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
        const uint16_t b = (c & 1) ? uint16_t(w >> 16) : uint16_t(w & 0xffffu);
        return (float)__builtin_bit_cast(_Float16, b);
    }
};
// fp16 halves of a key + tail group
__device__ __forceinline__ float f16_of(uint32_t w, int hi)
{
    return (float)__builtin_bit_cast(_Float16, uint16_t(hi ? (w >> 16) : (w & 0xffffu)));
}
template <int NC> struct HpStep<false, NC> {
    float4 a[NC];
    __device__ __forceinline__ void load(const void *base, int node, int cb, int C)
    {
        const float *nb = reinterpret_cast<const float *>(base) + (size_t)node * NC * C + cb;
#pragma unroll
        for (int e = 0; e < NC; ++e) a[e] = *reinterpret_cast<const float4 *>(nb + e * C);
    }
    __device__ __forceinline__ float get(int e, int c) const
    {
        const float4 &v = a[e];
        return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
    }
};

template <int N> struct Log2;
template <> struct Log2<1> { static constexpr int v = 0; };
template <> struct Log2<2> { static constexpr int v = 1; };
template <> struct Log2<4> { static constexpr int v = 2; };
template <> struct Log2<8> { static constexpr int v = 3; };

__device__ __forceinline__ float pick4(const floatx4 &v, int r)
{
    return r == 0 ? v[0] : r == 1 ? v[1] : r == 2 ? v[2] : v[3];
}

// Two targets per wave over the union of their lists (attn_pair.hip): 16-bit
// storage, l_max <= 2, n < attn_pair_max_atoms().
hipError_t launch_attn_pair(int L, const AttnArgs &a, hipStream_t stream);
int attn_pair_max_atoms();

}  // namespace e2v2
