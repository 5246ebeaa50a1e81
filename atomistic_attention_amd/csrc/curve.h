// The targets' Hilbert-curve processing order: device pieces shared by the
// neighbour builder (which emits the order beside the lists) and the standalone
// order call.
//
// The curve: the bounding box of the finite coordinates is cut into cubic cells
// of side 2^k, the largest power of two with 8 n (2^k)^3 <= V (V the box volume,
// each side at least 2^-10 of the longest, so a flat system still has a volume),
// raised if needed until the longest side holds fewer than 1023 cells.  Cell
// coordinates q = floor((p - lo) 2^-k) (clamped to 0..1023; NaN gives 0) go
// through the transposed form of the Hilbert index (J. Skilling, "Programming
// the Hilbert curve", AIP Conf. Proc. 707, 2004) with 10 bits per axis, and the
// atoms are sorted by (index, atom id), so the order is deterministic.  The
// occupied corner [0, 2^j)^3 of the 1024^3 grid is itself one Hilbert curve of
// order j, since the curve fills its first octant first at every level: every
// index is below 2^(3j).
//
// The sort: atoms counted into 4,096 buckets (the top 12 bits of the 3j-bit
// index, each an aligned block of cells); one workgroup scans the counts into
// bucket offsets and lists the work items (bucket, run of 64 entries); each atom
// takes a slot in its bucket by an atomic; one wave per work item ranks its
// entries within the bucket by counting the smaller (index, id) pairs, and the
// rank places the atom.  Buckets hold n / 4096 atoms on average at uniform
// density; a bucket holding most atoms (all in one small region beside a far
// outlier) costs time proportional to its size squared over 64, spread over its
// waves.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace e2v2 {
namespace curve {

constexpr int kCurveBits = 10;       // bits per axis of the Hilbert index
constexpr int kBucketBits = 12;
constexpr int kBuckets = 1 << kBucketBits;
constexpr int kRun = 64;             // entries ranked by one wave

struct CurveInfo {
    float lo[3];
    float inv;                       // 2^-k, or 0 when the box has no extent
    int shift;                       // bucket = index >> shift
    int pad[3];
};

inline long long max_items(int n) { return kBuckets + ((long long)n + kRun - 1) / kRun + 1; }

// Hilbert index of cell (x, y, z), kCurveBits bits per axis: the axes are turned
// into the curve's transposed form (Skilling's inverse of the excess work, then a
// Gray code), whose bits, read from the top level down and axis by axis, are the
// index.
__device__ __forceinline__ uint32_t hilbert_index(uint32_t x, uint32_t y, uint32_t z)
{
    uint32_t X[3] = {x, y, z};
    for (uint32_t Q = 1u << (kCurveBits - 1); Q > 1u; Q >>= 1) {
        const uint32_t P = Q - 1u;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (X[i] & Q) {
                X[0] ^= P;                               // invert the low bits
            } else {
                const uint32_t t = (X[0] ^ X[i]) & P;    // exchange the low bits
                X[0] ^= t;
                X[i] ^= t;
            }
        }
    }
    X[1] ^= X[0];
    X[2] ^= X[1];
    uint32_t t = 0;
    for (uint32_t Q = 1u << (kCurveBits - 1); Q > 1u; Q >>= 1)
        if (X[2] & Q) t ^= Q - 1u;
    X[0] ^= t;
    X[1] ^= t;
    X[2] ^= t;
    uint32_t key = 0;
    for (int j = kCurveBits - 1; j >= 0; --j)
#pragma unroll
        for (int i = 0; i < 3; ++i) key = (key << 1) | ((X[i] >> j) & 1u);
    return key;
}

// The cells from the box of the finite coordinates (lo = +inf, hi = -inf on an
// axis without any) of n atoms.
__device__ inline CurveInfo curve_setup(const float (&lo)[3], const float (&hi)[3], int n)
{
    CurveInfo c{};
    float ext[3], mx = 0.f;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        ext[a] = hi[a] - lo[a];
        mx = fmaxf(mx, ext[a]);
        c.lo[a] = std::isfinite(lo[a]) ? lo[a] : 0.f;
    }
    float iv = 0.f;                       // no extent (or none finite): every index 0
    if (mx > 0.f && std::isfinite(mx)) {
        const float fl = mx * 0x1p-10f;
        const double V = (double)fmaxf(ext[0], fl) * (double)fmaxf(ext[1], fl) * (double)fmaxf(ext[2], fl);
        int E = 0;
        frexp(V / (8.0 * (double)n), &E);            // V / (8 n) in [2^(E-1), 2^E)
        const int e1 = E - 1;
        int k = e1 >= 0 ? e1 / 3 : -((2 - e1) / 3);   // floor((E - 1) / 3)
        if (k < -126) k = -126;
        while (k < 127 && mx * ldexpf(1.f, -k) >= 1023.f) ++k;
        iv = ldexpf(1.f, -k);
    }
    c.inv = iv;
    // bits of the largest cell coordinate: every index is below 2^(3 j)
    const float cm = mx * iv;
    const uint32_t qm = cm >= 1023.f ? 1023u : (cm > 0.f ? (uint32_t)cm : 0u);
    const int j = qm > 0u ? 32 - __clz(qm) : 1;
    c.shift = 3 * j > kBucketBits ? 3 * j - kBucketBits : 0;
    return c;
}

__device__ __forceinline__ uint32_t curve_key(const CurveInfo &c, float x, float y, float z)
{
    const float p[3] = {x, y, z};
    uint32_t q[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const float v = (p[a] - c.lo[a]) * c.inv;
        q[a] = v >= 1023.f ? 1023u : (v > 0.f ? (uint32_t)v : 0u);   // NaN -> 0
    }
    return hilbert_index(q[0], q[1], q[2]);
}

__device__ __forceinline__ int bucket_of(uint32_t key, int shift)
{
    const uint32_t b = key >> shift;
    return b < (uint32_t)kBuckets ? (int)b : kBuckets - 1;     // monotone in the key
}

// Bucket offsets, slot cursors and the work list (bucket, run), by one workgroup
// of NTH threads.
template <int NTH>
__device__ inline void bucket_scan_block(const int32_t *__restrict__ cnt, int32_t *__restrict__ bstart,
                                         int32_t *__restrict__ cursor, int2 *__restrict__ items,
                                         int32_t *__restrict__ nitems)
{
    static_assert(kBuckets % NTH == 0, "whole buckets per thread");
    constexpr int PER = kBuckets / NTH;
    __shared__ int sa[NTH], sb[NTH];
    const int t = threadIdx.x;
    int c[PER], r[PER], ta = 0, tb = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        c[u] = cnt[PER * t + u];
        r[u] = (c[u] + kRun - 1) / kRun;
        ta += c[u];
        tb += r[u];
    }
    sa[t] = ta;
    sb[t] = tb;
    __syncthreads();
    for (int d = 1; d < NTH; d <<= 1) {           // inclusive scans of both totals
        const int xa = t >= d ? sa[t - d] : 0, xb = t >= d ? sb[t - d] : 0;
        __syncthreads();
        sa[t] += xa;
        sb[t] += xb;
        __syncthreads();
    }
    int oa = sa[t] - ta, ob = sb[t] - tb;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int b = PER * t + u;
        bstart[b] = oa;
        cursor[b] = oa;
        for (int k = 0; k < r[u]; ++k) items[ob + k] = make_int2(b, k);
        oa += c[u];
        ob += r[u];
    }
    if (t == NTH - 1) {
        bstart[kBuckets] = oa;
        *nitems = ob;
    }
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work item w (one wave, lane 0..63, tile a wave-private LDS array of kRun): the
// rank of each of its entries among the bucket's (index, id) pairs, all
// distinct, places the atom.  Items at or past *nitems do nothing.
__device__ inline void rank_item(const uint64_t *__restrict__ ent, const int32_t *__restrict__ bstart,
                                 const int2 *__restrict__ items, const int32_t *__restrict__ nitems, long long w,
                                 int lane, uint64_t *tile, int32_t *__restrict__ order)
{
    if (w >= *nitems) return;
    const int2 it = items[w];
    const int base = bstart[it.x], m = bstart[it.x + 1] - base;
    const int e = it.y * kRun + lane;
    const uint64_t v = e < m ? ent[base + e] : ~uint64_t(0);
    int rank = 0;
    for (int t0 = 0; t0 < m; t0 += kRun) {
        const int u = t0 + lane;
        tile[lane] = u < m ? ent[base + u] : ~uint64_t(0);
        wave_lds_sync();
        const int lim = min(kRun, m - t0);
        for (int k = 0; k < lim; ++k) rank += tile[k] < v ? 1 : 0;
        wave_lds_sync();
    }
    if (e < m) order[base + rank] = (int32_t)(uint32_t)v;
}

}  // namespace curve
}  // namespace e2v2
