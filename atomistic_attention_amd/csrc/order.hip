// The standalone call for the targets' Hilbert-curve processing order
// (e2v2_target_order): the curve and its sort are described in curve.h; here they
// run in five launches with no host work between them: (1) partial bounding
// boxes, which also clear the bucket counts; (2) the cells, each atom's index and
// its bucket count; (3) the bucket scan and work list; (4) the slots; (5) the
// ranks.
#include "curve.h"
#include "e2v2_internal.h"

namespace e2v2 {

namespace {

using namespace curve;

constexpr int kOrderParts = 256;     // blocks of the bounding-box pass (at most)

struct OrderLayout {
    float *part;          // [kOrderParts][6] partial (min, max) per axis
    int32_t *cnt;         // [kBuckets] atoms per bucket
    int32_t *bstart;      // [kBuckets + 1] bucket offsets
    int32_t *cursor;      // [kBuckets] next free slot per bucket
    CurveInfo *info;      // the cells (written by every block of step 2, block 0's kept)
    int32_t *nitems;      // [1] work items listed
    int2 *items;          // [max_items(n)] (bucket, run)
    uint32_t *key;        // [n] Hilbert indices
    uint64_t *ent;        // [n] (index << 32 | atom id), grouped by bucket
    size_t bytes;
};

inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

OrderLayout order_layout(void *ws, int n)
{
    OrderLayout L{};
    char *p = reinterpret_cast<char *>(ws);
    size_t o = 0;
    L.part = reinterpret_cast<float *>(p + o); o += al256(sizeof(float) * 6 * kOrderParts);
    L.cnt = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * kBuckets);
    L.bstart = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (kBuckets + 1));
    L.cursor = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * kBuckets);
    L.info = reinterpret_cast<CurveInfo *>(p + o); o += al256(sizeof(CurveInfo));
    L.nitems = reinterpret_cast<int32_t *>(p + o); o += 256;
    L.items = reinterpret_cast<int2 *>(p + o); o += al256(sizeof(int2) * (size_t)max_items(n));
    L.key = reinterpret_cast<uint32_t *>(p + o); o += al256(sizeof(uint32_t) * (size_t)n);
    L.ent = reinterpret_cast<uint64_t *>(p + o); o += al256(sizeof(uint64_t) * (size_t)n);
    L.bytes = o;
    return L;
}

// (1) Per block: min and max of the finite coordinates of a strided slice of
// atoms; the blocks also clear the bucket counts.
__global__ __launch_bounds__(256) void k_order_bbox(const float *__restrict__ pos, int n, float *__restrict__ part,
                                                    int32_t *__restrict__ cnt)
{
    __shared__ float s[6][256];
    const int t = threadIdx.x;
    for (int b = blockIdx.x * 256 + t; b < kBuckets; b += gridDim.x * 256) cnt[b] = 0;
    float lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
    for (long long i = (long long)blockIdx.x * 256 + t; i < n; i += (long long)gridDim.x * 256) {
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            const float v = pos[3 * i + a];
            if (std::isfinite(v)) {
                lo[a] = fminf(lo[a], v);
                hi[a] = fmaxf(hi[a], v);
            }
        }
    }
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        s[a][t] = lo[a];
        s[3 + a][t] = hi[a];
    }
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) {
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                s[a][t] = fminf(s[a][t], s[a][t + w]);
                s[3 + a][t] = fmaxf(s[3 + a][t], s[3 + a][t + w]);
            }
        }
        __syncthreads();
    }
    if (t < 6) part[blockIdx.x * 6 + t] = s[t][0];
}

// (2) Every block combines the partial boxes and sizes the cells (the same
// arithmetic in every block), then writes its atoms' indices and counts them per
// bucket.
__global__ __launch_bounds__(256) void k_order_keys(const float *__restrict__ pos, int n,
                                                    const float *__restrict__ part, int nparts,
                                                    uint32_t *__restrict__ key, int32_t *__restrict__ cnt,
                                                    CurveInfo *__restrict__ info)
{
    __shared__ float s[6][256];
    __shared__ CurveInfo ci;
    const int t = threadIdx.x;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        s[a][t] = t < nparts ? part[6 * t + a] : INFINITY;
        s[3 + a][t] = t < nparts ? part[6 * t + 3 + a] : -INFINITY;
    }
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) {
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                s[a][t] = fminf(s[a][t], s[a][t + w]);
                s[3 + a][t] = fmaxf(s[3 + a][t], s[3 + a][t + w]);
            }
        }
        __syncthreads();
    }
    if (t == 0) {
        const float lo[3] = {s[0][0], s[1][0], s[2][0]}, hi[3] = {s[3][0], s[4][0], s[5][0]};
        ci = curve_setup(lo, hi, n);
        if (blockIdx.x == 0) *info = ci;
    }
    __syncthreads();
    const long long i = (long long)blockIdx.x * 256 + t;
    if (i >= n) return;
    const uint32_t k = curve_key(ci, pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]);
    key[i] = k;
    atomicAdd(&cnt[bucket_of(k, ci.shift)], 1);
}

// (3) Bucket offsets, slot cursors and the work list.
__global__ __launch_bounds__(1024) void k_order_scan(const int32_t *__restrict__ cnt, int32_t *__restrict__ bstart,
                                                     int32_t *__restrict__ cursor, int2 *__restrict__ items,
                                                     int32_t *__restrict__ nitems)
{
    bucket_scan_block<1024>(cnt, bstart, cursor, items, nitems);
}

// (4) Each atom takes a slot in its bucket.
__global__ __launch_bounds__(256) void k_order_scatter(const uint32_t *__restrict__ key, int n,
                                                       const CurveInfo *__restrict__ info,
                                                       int32_t *__restrict__ cursor, uint64_t *__restrict__ ent)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint32_t k = key[i];
    const int slot = atomicAdd(&cursor[bucket_of(k, info->shift)], 1);
    ent[slot] = (uint64_t(k) << 32) | uint32_t(i);
}

// (5) One wave per work item.
__global__ __launch_bounds__(64) void k_order_rank(const uint64_t *__restrict__ ent,
                                                   const int32_t *__restrict__ bstart,
                                                   const int2 *__restrict__ items, const int32_t *__restrict__ nitems,
                                                   int32_t *__restrict__ order)
{
    __shared__ uint64_t tile[kRun];
    rank_item(ent, bstart, items, nitems, blockIdx.x, threadIdx.x, tile, order);
}

}  // namespace

size_t target_order_ws_bytes(int n) { return order_layout(nullptr, n < 1 ? 1 : n).bytes; }

hipError_t launch_target_order(const float *pos, int n, void *ws, int32_t *order, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    OrderLayout L = order_layout(ws, n);
    const int nparts = (int)std::min<long long>(kOrderParts, ((long long)n + 255) / 256);
    const unsigned nb = (unsigned)(((long long)n + 255) / 256);
    k_order_bbox<<<nparts, 256, 0, stream>>>(pos, n, L.part, L.cnt);
    k_order_keys<<<nb, 256, 0, stream>>>(pos, n, L.part, nparts, L.key, L.cnt, L.info);
    k_order_scan<<<1, 1024, 0, stream>>>(L.cnt, L.bstart, L.cursor, L.items, L.nitems);
    k_order_scatter<<<nb, 256, 0, stream>>>(L.key, n, L.info, L.cursor, L.ent);
    k_order_rank<<<(unsigned)max_items(n), kRun, 0, stream>>>(L.ent, L.bstart, L.items, L.nitems, order);
    return hipGetLastError();
}

}  // namespace e2v2
