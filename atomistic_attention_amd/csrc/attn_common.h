// Helpers shared by the streaming attention kernels (attn.hip, attn_pair.hip):
// the per-lane value-row pieces and small lane utilities.
#pragma once

#include "e2v2_internal.h"

namespace e2v2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// One neighbour's value pieces for this lane's 4 channels.  16-bit h' is stored with
// components interleaved in pairs (hp_f16_offset): one 16-byte load covers 4
// channels of two components -- half the load instructions of a per-component
// layout -- and an odd last component is one more 8-byte load (hp_row16).
template <bool HB, int NC> struct HpStep;
template <int NC> struct HpStep<true, NC> {
    static constexpr int NPR = NC / 2;
    static constexpr bool ODD = (NC & 1) != 0;
    uint4 pr[NPR > 0 ? NPR : 1];
    uint2 tl;                                    // the odd last component (odd NC)
    __device__ __forceinline__ void load(const void *base, int node, int cb, int C)
    {
        const uint16_t *nb = reinterpret_cast<const uint16_t *>(base) + (size_t)node * hp_row16(NC, C);
#pragma unroll
        for (int p = 0; p < NPR; ++p) pr[p] = *reinterpret_cast<const uint4 *>(nb + p * 2 * C + (cb >> 2) * 8);
        if constexpr (ODD) tl = *reinterpret_cast<const uint2 *>(nb + (NC - 1) * C + cb);
    }
    // The same row addressed by a 32-bit byte offset from base (row * row bytes
    // must stay below 2^32): one scalar base plus one 32-bit offset per load.
    __device__ __forceinline__ void load32(const void *base, uint32_t row, int cb, int C)
    {
        const unsigned char *rb = reinterpret_cast<const unsigned char *>(base) + row * uint32_t(2 * hp_row16(NC, C));
        const unsigned char *nb = rb + uint32_t(cb >> 2) * 16u;
#pragma unroll
        for (int p = 0; p < NPR; ++p) pr[p] = *reinterpret_cast<const uint4 *>(nb + p * 4 * C);
        if constexpr (ODD) tl = *reinterpret_cast<const uint2 *>(rb + uint32_t(2 * (NC - 1) * C + 2 * cb));
    }
    // component e, channel c of the lane's 4
    __device__ __forceinline__ float get(int e, int c) const
    {
        if (ODD && e == NC - 1) {
            const uint32_t w = c < 2 ? tl.x : tl.y;
            return (float)__builtin_bit_cast(_Float16, uint16_t((c & 1) ? (w >> 16) : (w & 0xffffu)));
        }
        const uint4 &v = pr[e >> 1];
        const int k = (e & 1) * 2 + (c >> 1);
        const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
        const uint16_t b = (c & 1) ? uint16_t(w >> 16) : uint16_t(w & 0xffffu);
        return (float)__builtin_bit_cast(_Float16, b);
    }
};
// fp16 halves of a 32-bit word
__device__ __forceinline__ float f16_of(uint32_t w, int hi)
{
    return (float)__builtin_bit_cast(_Float16, uint16_t(hi ? (w >> 16) : (w & 0xffffu)));
}

template <int N> struct Log2;
template <> struct Log2<1> { static constexpr int v = 0; };
template <> struct Log2<2> { static constexpr int v = 1; };
template <> struct Log2<4> { static constexpr int v = 2; };
template <> struct Log2<8> { static constexpr int v = 3; };

__device__ __forceinline__ float pick4(const floatx4 &v, int r)
{
    return r == 0 ? v[0] : r == 1 ? v[1] : r == 2 ? v[2] : v[3];
}

// Stores one target's normalised message m_i after the slot merge (16-bit
// storage): lane holds channels cb + off + c, c < NCH, of every component in
// acc (not yet divided by z).  m_i is written in fp16 under one power-of-two
// scale per node -- the largest |m_i| M below 2^14 s, the rule the source
// features use -- and s goes to A.msc[i]; the tap receives the stored values.
template <int NC, int NCH>
__device__ __forceinline__ void store_message_f16(const AttnArgs &A, int i, int C, float z, const float (&acc)[NC][4],
                                                  int ch0, bool writer, int lane)
{
    const float invz = z > 0.f ? 1.f / z : 0.f;
    unsigned mb = 0u;
#pragma unroll
    for (int e = 0; e < NC; ++e)
#pragma unroll
        for (int c = 0; c < NCH; ++c) mb = max(mb, __float_as_uint(acc[e][c] * invz) & 0x7fffffffu);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mb = max(mb, (unsigned)__shfl_xor((int)mb, d, 64));
    unsigned sb = 127u;                                  // scale 1 for zero or non-finite rows
    if (mb != 0u && mb < 0x7f800000u) {
        const unsigned b = mb >> 23;
        sb = b > 13u ? b - 13u : 1u;
    }
    const float sc = __uint_as_float(sb << 23), inv = __uint_as_float((254u - sb) << 23);
    if (lane == 0) A.msc[i] = sc;
    if (!writer) return;
#pragma unroll
    for (int e = 0; e < NC; ++e) {
        const size_t o = ((size_t)i * NC + e) * C + ch0;
        _Float16 hv[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) hv[c] = (_Float16)(acc[e][c] * invz * inv);
        if constexpr (NCH == 2) {
            *reinterpret_cast<uint32_t *>(A.mh + o) =
                uint32_t(__builtin_bit_cast(uint16_t, hv[0])) | (uint32_t(__builtin_bit_cast(uint16_t, hv[1])) << 16);
        } else {
#pragma unroll
            for (int c = 0; c < NCH; ++c) A.mh[o + c] = __builtin_bit_cast(uint16_t, hv[c]);
        }
        if (A.m_tap) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) A.m_tap[o + c] = (float)hv[c] * sc;
        }
    }
}

// Two targets per wave over the union of their lists (attn_pair.hip): 16-bit
// storage, l_max <= 2, n < attn_pair_max_atoms(L, C).
hipError_t launch_attn_pair(int L, const AttnArgs &a, hipStream_t stream);
long long attn_pair_max_atoms(int L, int C);
// Four targets per wave, weighted sums on the matrix cores (attn_quad.hip): h' in
// hp_quad_offset layout, hp_quad_layout(L, H, C, n) must hold.
hipError_t launch_attn_quad(int L, const AttnArgs &a, hipStream_t stream);

}  // namespace e2v2
