// Cell-list neighbour list (E2Former-V2 explainer, section 3.2: a neighbour cap
// K with masked padding; section 5.2: the list must be right).  Every candidate
// pair is decided by the fp64 predicate
//     dx = (double)x_j - (double)x_i  (likewise dy, dz),
//     d2 = (dx*dx + dy*dy) + dz*dz < (double)cutoff^2,
// with no fused multiply-add, so the result is bit-identical to a brute-force
// search with the same arithmetic.
//
// Steps (all on the caller's stream):
//   1. partial bounding boxes;
//   2. every block combines them and sizes a grid whose cells are about half the
//      cutoff wide (at most n + 64 cells); cell index per atom + per-cell counts
//      (integer atomics: counts are exact);
//   3. exclusive scan of the counts; scatter atoms into cell order;
//   4. one wave per target (targets taken in cell order, so neighbouring waves
//      read the same cells) visits the rows of cells that the cutoff sphere can
//      reach, each row cut along x to the sphere's extent there (so the scan
//      covers little more than the sphere), compacts the pairs that pass into
//      LDS and writes them in the scan's order (rows of cells by z, then y; the
//      cells of a row in index order; atoms ascending within a cell):
//        K = 0: count -> scan -> fill;
//        K > 0: padded with -1; a row with more than K candidates keeps the K
//               nearest by (d2, j), in that order (a register bitonic sort of the
//               (d2, j) keys).
//      Rows with more candidates than the LDS buffer holds are filled by lane 0
//      of their wave alone (a max-heap held in the row itself, then a heapsort:
//      those rows ascend by j).
//   The reach of the sphere along each axis is widened by a margin that covers
//   fp32 rounding in the cell index and the cell bounds, so the rows and cells
//   visited are always a superset of the ones holding a neighbour.
// Atoms are ranked by index within a cell after the atomic scatter and the
// K-nearest choice uses a total order, so rows and their order are deterministic.
#include "curve.h"
#include "e2v2_internal.h"

#include <algorithm>

#pragma clang fp contract(off)

namespace e2v2 {

struct GridInfo {
    float lo[3];
    float inv[3];          // cells per unit length (cell index = floor((x - lo) * inv), clamped)
    float w[3];            // cell width
    float margin;          // widening of every reach test: covers fp32 rounding of bounds and indices
    int dims[3];
    int ncell;
};

struct NbrLayout {
    GridInfo *grid;
    float *box_part;       // [kBoxBlocks][16] partial bounding boxes: all values (min 0..2,
                           // max 4..6), finite values (min 8..10, max 12..14)
    int32_t *cell_of;
    int32_t *cell_cnt;     // [maxc + 1]
    int32_t *cell_start;   // [maxc + 1]
    int32_t *cell_cur;     // [maxc]
    int32_t *order;        // [n] atom ids in cell order
    float4 *spos;          // [n] positions in cell order, w = atom id bits
    int64_t *nnz;
    int32_t *mval;         // [n] the atomic slots of the cell scatter
    // the Hilbert processing order (curve.h), when the caller asks for it
    curve::CurveInfo *curve;
    int32_t *bcnt, *bstart, *bcursor, *nitems;   // [kBuckets], [kBuckets + 1], [kBuckets], [1]
    int2 *items;           // [max_items(n)]
    uint32_t *key;         // [n]
    uint64_t *ent;         // [n]
    size_t bytes;
};

static inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
static inline int max_cells(int n) { return n + 64; }

static NbrLayout nbr_layout(void *ws, int n)
{
    NbrLayout L{};
    char *p = reinterpret_cast<char *>(ws);
    size_t o = 0;
    const size_t mc = (size_t)max_cells(n);
    L.grid = reinterpret_cast<GridInfo *>(p + o); o += al256(sizeof(GridInfo));
    L.box_part = reinterpret_cast<float *>(p + o); o += al256(sizeof(float) * 16 * 256);
    L.nnz = reinterpret_cast<int64_t *>(p + o); o += al256(sizeof(int64_t));
    L.cell_of = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (size_t)n);
    L.cell_cnt = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (mc + 1));
    L.cell_start = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (mc + 1));
    L.cell_cur = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * mc);
    L.order = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (size_t)n);
    L.spos = reinterpret_cast<float4 *>(p + o); o += al256(sizeof(float4) * (size_t)n);
    L.mval = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (size_t)n);
    L.curve = reinterpret_cast<curve::CurveInfo *>(p + o); o += al256(sizeof(curve::CurveInfo));
    L.bcnt = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * curve::kBuckets);
    L.bstart = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * (curve::kBuckets + 1));
    L.bcursor = reinterpret_cast<int32_t *>(p + o); o += al256(sizeof(int32_t) * curve::kBuckets);
    L.nitems = reinterpret_cast<int32_t *>(p + o); o += 256;
    L.items = reinterpret_cast<int2 *>(p + o); o += al256(sizeof(int2) * (size_t)curve::max_items(n));
    L.key = reinterpret_cast<uint32_t *>(p + o); o += al256(sizeof(uint32_t) * (size_t)n);
    L.ent = reinterpret_cast<uint64_t *>(p + o); o += al256(sizeof(uint64_t) * (size_t)n);
    L.bytes = o;
    return L;
}

size_t neighbors_ws_bytes(int n, int /*K*/) { return nbr_layout(nullptr, n).bytes; }
int64_t *neighbors_nnz_slot(void *ws, int n) { return nbr_layout(ws, n).nnz; }

// ---------------------------------------------------------------- step 1
// Bounding box in two stages: kBoxBlocks blocks reduce strided slices into
// partial (min, max) records (and clear the cell counters for step 2); every block
// of step 2 combines them and sizes the grid.
constexpr int kBoxBlocks = 256;

__global__ __launch_bounds__(256) void k_bbox_partial(const float *__restrict__ pos, int n, float *part, int maxc,
                                                      int32_t *cell_cnt, int32_t *bcnt)
{
    __shared__ float sv[12][256];      // min 0..2, max 3..5 over all values; 6..8, 9..11 over finite ones
    const int t = threadIdx.x;
    for (long long c = (long long)blockIdx.x * 256 + t; c <= maxc; c += (long long)gridDim.x * 256) cell_cnt[c] = 0;
    if (bcnt)
        for (int b = blockIdx.x * 256 + t; b < curve::kBuckets; b += gridDim.x * 256) bcnt[b] = 0;
    float v[12];
    for (int d = 0; d < 3; ++d) {
        v[d] = v[6 + d] = INFINITY;
        v[3 + d] = v[9 + d] = -INFINITY;
    }
    for (long long i = (long long)blockIdx.x * 256 + t; i < n; i += (long long)gridDim.x * 256)
        for (int d = 0; d < 3; ++d) {
            const float x = pos[3 * i + d];
            v[d] = fminf(v[d], x);       // fminf/fmaxf ignore NaN
            v[3 + d] = fmaxf(v[3 + d], x);
            if (std::isfinite(x)) {
                v[6 + d] = fminf(v[6 + d], x);
                v[9 + d] = fmaxf(v[9 + d], x);
            }
        }
    for (int q = 0; q < 12; ++q) sv[q][t] = v[q];
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s)
            for (int d = 0; d < 3; ++d) {
                sv[d][t] = fminf(sv[d][t], sv[d][t + s]);
                sv[3 + d][t] = fmaxf(sv[3 + d][t], sv[3 + d][t + s]);
                sv[6 + d][t] = fminf(sv[6 + d][t], sv[6 + d][t + s]);
                sv[9 + d][t] = fmaxf(sv[9 + d][t], sv[9 + d][t + s]);
            }
        __syncthreads();
    }
    if (t < 3) {
        part[blockIdx.x * 16 + t] = sv[t][0];
        part[blockIdx.x * 16 + 4 + t] = sv[3 + t][0];
        part[blockIdx.x * 16 + 8 + t] = sv[6 + t][0];
        part[blockIdx.x * 16 + 12 + t] = sv[9 + t][0];
    }
}

// One block of 256 threads: the grid from the partial boxes and, when asked for,
// the cells of the Hilbert processing order from the finite values' box (grid and
// cinfo may point to LDS; every block that calls it does the same arithmetic).
__device__ inline void grid_setup_block(const float *__restrict__ part, int nparts, float cutoff, int maxc,
                                        GridInfo *grid, int n, curve::CurveInfo *cinfo)
{
    __shared__ float sv[12][256];
    const int t = threadIdx.x;
    for (int d = 0; d < 3; ++d) {
        sv[d][t] = t < nparts ? part[t * 16 + d] : INFINITY;
        sv[3 + d][t] = t < nparts ? part[t * 16 + 4 + d] : -INFINITY;
        sv[6 + d][t] = t < nparts ? part[t * 16 + 8 + d] : INFINITY;
        sv[9 + d][t] = t < nparts ? part[t * 16 + 12 + d] : -INFINITY;
    }
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s)
            for (int d = 0; d < 3; ++d) {
                sv[d][t] = fminf(sv[d][t], sv[d][t + s]);
                sv[3 + d][t] = fmaxf(sv[3 + d][t], sv[3 + d][t + s]);
                sv[6 + d][t] = fminf(sv[6 + d][t], sv[6 + d][t + s]);
                sv[9 + d][t] = fmaxf(sv[9 + d][t], sv[9 + d][t + s]);
            }
        __syncthreads();
    }
    if (t == 1 && cinfo) {
        const float lo[3] = {sv[6][0], sv[7][0], sv[8][0]}, hi[3] = {sv[9][0], sv[10][0], sv[11][0]};
        *cinfo = curve::curve_setup(lo, hi, n);
    }
    if (t == 0) {
        float smin[3], smax[3];
        for (int d = 0; d < 3; ++d) {
            smin[d] = sv[d][0];
            smax[d] = sv[3 + d][0];
        }
        const float cmin = 0.5f * cutoff * 1.001f;              // two cells per cutoff
        int dims[3];
        float ext[3];
        for (int d = 0; d < 3; ++d) {
            ext[d] = smax[d] - smin[d];
            float k = (ext[d] < 1e30f) ? floorf(ext[d] / cmin) : 1.f;   // false for NaN / inf
            dims[d] = (k >= 1.f) ? (int)fminf(k, 1024.f) : 1;
        }
        while ((long long)dims[0] * dims[1] * dims[2] > maxc) {
            int a = 0;
            if (dims[1] > dims[a]) a = 1;
            if (dims[2] > dims[a]) a = 2;
            dims[a] = dims[a] * 7 / 8 > 0 ? dims[a] * 7 / 8 : 1;
        }
        float mag = 0.f;
        for (int d = 0; d < 3; ++d) {
            grid->lo[d] = (smin[d] < 1e30f && smin[d] > -1e30f) ? smin[d] : 0.f;
            grid->inv[d] = dims[d] > 1 ? (float)dims[d] / ext[d] : 0.f;
            grid->w[d] = dims[d] > 1 ? ext[d] / (float)dims[d] : INFINITY;
            grid->dims[d] = dims[d];
            mag = fmaxf(mag, fmaxf(fabsf(smin[d]), fabsf(smax[d])));
        }
        // fp32 rounding of a coordinate-sized quantity is below 6e-8 of the largest
        // coordinate; 1e-5 of it (plus 1e-4 of the cutoff) is a wide bound
        const float m = 1e-5f * mag + 1e-4f * cutoff;
        grid->margin = (m < 1e30f) ? m : INFINITY;              // NaN / inf: every cell is in reach
        grid->ncell = dims[0] * dims[1] * dims[2];
    }
}

__device__ __forceinline__ int cell_coord(float x, float lo, float inv, int dim)
{
    const float t = (x - lo) * inv;
    if (!(t > 0.f)) return 0;                                // also NaN
    return t >= (float)(dim - 1) ? dim - 1 : (int)t;
}

// Cells [c0, c1] along axis d that hold every coordinate within r of p.  Cell
// indices are monotone in the coordinate, so the ends' cells bound them.
__device__ __forceinline__ void axis_reach(float p, float r, const GridInfo &gi, int d, int &c0, int &c1)
{
    c0 = cell_coord(p - r, gi.lo[d], gi.inv[d], gi.dims[d]);
    c1 = cell_coord(p + r, gi.lo[d], gi.inv[d], gi.dims[d]);
}

// Distance along axis d from p to the coordinates of cell c (the first and last
// cells reach to -inf / +inf), reduced by the margin: never more than the true gap.
__device__ __forceinline__ float axis_gap(float p, int c, const GridInfo &gi, int d)
{
    const float a = c > 0 ? gi.lo[d] + (float)c * gi.w[d] : -INFINITY;
    const float b = c < gi.dims[d] - 1 ? gi.lo[d] + (float)(c + 1) * gi.w[d] : INFINITY;
    const float g = fmaxf(fmaxf(a - p, p - b), 0.f);         // fmaxf drops a NaN operand
    return fmaxf(g - gi.margin, 0.f);
}

// The x-cells of row (z, y) that a sphere of radius rcm about p can reach, as
// [x0, x1]; false if the row is out of reach.
__device__ __forceinline__ bool row_reach(float4 p, float rcm, int z, int y, const GridInfo &gi, int &x0, int &x1)
{
    const float gz = axis_gap(p.z, z, gi, 2), gy = axis_gap(p.y, y, gi, 1);
    const float rem = rcm * rcm - gz * gz - gy * gy;
    if (!(rem > 0.f)) return false;
    axis_reach(p.x, sqrtf(rem) + gi.margin, gi, 0, x0, x1);
    return true;
}

// Cells are numbered in serpentine order: z-planes in turn, the rows of every odd
// plane in reverse y order, and every odd row (counting rows globally) in reverse
// x order.  Consecutive cells stay adjacent in space across row and plane ends,
// so the cell order is a processing order whose runs of targets are compact, and
// every row of cells is still one contiguous index range.
__device__ __forceinline__ int row_base(const GridInfo &gi, int z, int y, bool &rev)
{
    const int ys = (z & 1) ? gi.dims[1] - 1 - y : y;
    const int row = z * gi.dims[1] + ys;
    rev = (row & 1) != 0;
    return row * gi.dims[0];
}
__device__ __forceinline__ int cell_index(const GridInfo &gi, int cx, int cy, int cz)
{
    bool rev;
    const int b = row_base(gi, cz, cy, rev);
    return b + (rev ? gi.dims[0] - 1 - cx : cx);
}
// Cells [lo, hi] (inclusive) holding x-cells x0 .. x1 of row (z, y).
__device__ __forceinline__ void row_cells(const GridInfo &gi, int z, int y, int x0, int x1, int &lo, int &hi)
{
    bool rev;
    const int b = row_base(gi, z, y, rev);
    lo = b + (rev ? gi.dims[0] - 1 - x1 : x0);
    hi = b + (rev ? gi.dims[0] - 1 - x0 : x1);
}

// ---------------------------------------------------------------- step 2
// Every block sizes the grid (and the curve's cells) from the partial boxes, block
// 0 stores them for the later steps; then each atom's cell and, when the
// processing order is asked for, its Hilbert index and bucket count.
__global__ __launch_bounds__(256) void k_cell_assign(const float *__restrict__ pos, int n,
                                                     const float *__restrict__ part, int nparts, float cutoff,
                                                     int maxc, GridInfo *grid, int32_t *cell_of, int32_t *cell_cnt,
                                                     curve::CurveInfo *cinfo_out, uint32_t *key, int32_t *bcnt)
{
    __shared__ GridInfo sg;
    __shared__ curve::CurveInfo sc;
    grid_setup_block(part, nparts, cutoff, maxc, &sg, n, cinfo_out ? &sc : nullptr);
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *grid = sg;
        if (cinfo_out) *cinfo_out = sc;
    }
    const curve::CurveInfo *cinfo = cinfo_out ? &sc : nullptr;
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const GridInfo gi = sg;
    const float x = pos[3 * i + 0], y = pos[3 * i + 1], z = pos[3 * i + 2];
    const int cx = cell_coord(x, gi.lo[0], gi.inv[0], gi.dims[0]);
    const int cy = cell_coord(y, gi.lo[1], gi.inv[1], gi.dims[1]);
    const int cz = cell_coord(z, gi.lo[2], gi.inv[2], gi.dims[2]);
    const int c = cell_index(gi, cx, cy, cz);
    cell_of[i] = c;
    atomicAdd(&cell_cnt[c], 1);
    if (cinfo) {
        const curve::CurveInfo ci = *cinfo;
        const uint32_t k = curve::curve_key(ci, x, y, z);
        key[i] = k;
        atomicAdd(&bcnt[curve::bucket_of(k, ci.shift)], 1);
    }
}

// Exclusive scan of in[0..count) into out[0..count], out[count] = total; one block
// of NTH threads.  If total_out is non-null the total is also stored there as
// int64.  The input is taken in tiles of 4 NTH: each thread sums 4 consecutive
// entries, the wave scans the sums with shuffles, the wave totals meet in LDS, and
// a carry runs from tile to tile; loads and stores stay coalesced.
template <int NTH>
__device__ inline void scan_block(const int32_t *__restrict__ in, const int *count_dev, int count_arg, int32_t *out,
                                  int32_t *copy, int64_t *total_out)
{
    constexpr int NW = NTH / 64;
    __shared__ long long wsum[NW];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int count = count_dev ? *count_dev : count_arg;
    long long carry = 0;
    for (long long base = 0; base < count; base += 4 * NTH) {
        const long long e0 = base + 4 * t;
        int v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (e0 + k < count) ? in[e0 + k] : 0;
        const long long sum = (long long)v[0] + v[1] + v[2] + v[3];
        long long x = sum;                                  // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const long long y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        long long before = 0, tile = 0;
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const long long ws = wsum[k];
            before += k < w ? ws : 0;
            tile += ws;
        }
        long long run = carry + before + x - sum;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (e0 + k < count) {
                out[e0 + k] = (int32_t)run;
                if (copy) copy[e0 + k] = (int32_t)run;
            }
            run += v[k];
        }
        carry += tile;
        __syncthreads();                                    // wsum is rewritten by the next tile
    }
    if (t == 0) {
        out[count] = (int32_t)carry;
        if (total_out) *total_out = carry;
    }
}

__global__ __launch_bounds__(1024) void k_scan(const int32_t *__restrict__ in, const int *count_dev, int count_arg,
                                               int32_t *out, int32_t *copy, int64_t *total_out)
{
    scan_block<1024>(in, count_dev, count_arg, out, copy, total_out);
}

// The cell scan (block 0) and the processing order's bucket scan (block 1) in one
// launch, in blocks of 256 threads: they then fit on a CU beside the blocks of a
// kernel running on another stream (the projections, in the two-stream step).
constexpr int kScanThreads = 256;
__global__ __launch_bounds__(kScanThreads) void k_scan_cells_buckets(const int32_t *__restrict__ cell_cnt, const int *ncell,
                                                             int32_t *cell_start, int32_t *cell_cur,
                                                             const int32_t *__restrict__ bcnt, int32_t *bstart,
                                                             int32_t *bcursor, int2 *items, int32_t *nitems)
{
    if (blockIdx.x == 0) scan_block<kScanThreads>(cell_cnt, ncell, 0, cell_start, cell_cur, nullptr);
    else curve::bucket_scan_block<kScanThreads>(bcnt, bstart, bcursor, items, nitems);
}

// ---------------------------------------------------------------- step 3
// Two passes, so the order within a cell does not depend on the timing of atomics:
// k_scatter drops every atom into its cell's range at an atomic slot (scratch),
// then k_place puts it at its rank by atom index within that range.  The cells
// follow the serpentine order of cell_index, and within a cell atoms ascend: the
// same order on every call.  A cell of k atoms costs k reads per atom.
__global__ void k_scatter(int n, const int32_t *__restrict__ cell_of, int32_t *cell_cur, int32_t *tmp,
                          const curve::CurveInfo *__restrict__ cinfo, const uint32_t *__restrict__ key,
                          int32_t *bcursor, uint64_t *ent)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int slot = atomicAdd(&cell_cur[cell_of[i]], 1);
    tmp[slot] = (int32_t)i;
    if (cinfo) {            // the atom's slot in its bucket of the processing order
        const uint32_t k = key[i];
        const int b = atomicAdd(&bcursor[curve::bucket_of(k, cinfo->shift)], 1);
        ent[b] = (uint64_t(k) << 32) | uint32_t(i);
    }
}
// Blocks below nplace place the atoms in cell order; the blocks after them, four
// waves each, rank the work items of the processing order (curve.h) into
// order_out.
__global__ __launch_bounds__(256) void k_place(const float *__restrict__ pos, int n,
                                               const int32_t *__restrict__ cell_of,
                                               const int32_t *__restrict__ cell_start,
                                               const int32_t *__restrict__ tmp, int32_t *order, float4 *spos,
                                               unsigned nplace, const uint64_t *__restrict__ ent,
                                               const int32_t *__restrict__ bstart, const int2 *__restrict__ items,
                                               const int32_t *__restrict__ nitems, int32_t *order_out)
{
    if (blockIdx.x >= nplace) {
        __shared__ uint64_t tile[4][curve::kRun];
        const int w = threadIdx.x >> 6;
        curve::rank_item(ent, bstart, items, nitems, 4LL * (blockIdx.x - nplace) + w, threadIdx.x & 63, tile[w],
                         order_out);
        return;
    }
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int c = cell_of[i];
    const int cs = cell_start[c], ce = cell_start[c + 1];
    int rank = 0;
    for (int t = cs; t < ce; ++t) rank += tmp[t] < (int32_t)i;
    const int slot = cs + rank;
    order[slot] = (int32_t)i;
    spos[slot] = make_float4(pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], __int_as_float((int)i));
}

// ---------------------------------------------------------------- step 4
__device__ __forceinline__ double pair_d2(double xi, double yi, double zi, float4 pj)
{
    const double dx = (double)pj.x - xi;
    const double dy = (double)pj.y - yi;
    const double dz = (double)pj.z - zi;
    const double xx = dx * dx;   // fp contract is off in this file: each op rounds
    const double yy = dy * dy;
    const double zz = dz * dz;
    const double s = xx + yy;
    return s + zz;
}
__device__ __forceinline__ double d2_of(const float *__restrict__ pos, double xi, double yi, double zi, int j)
{
    return pair_d2(xi, yi, zi, make_float4(pos[3 * (size_t)j], pos[3 * (size_t)j + 1], pos[3 * (size_t)j + 2], 0.f));
}

// Visits every candidate j != i within reach of the cutoff sphere with d2 < rc2.
template <typename F>
__device__ __forceinline__ void for_each_neighbor(int i, float4 pi, float rc, double rc2, const GridInfo &gi,
                                                  const int32_t *__restrict__ cell_start,
                                                  const float4 *__restrict__ spos, F &&f)
{
    const double xi = pi.x, yi = pi.y, zi = pi.z;
    const float rcm = rc + gi.margin;
    int z0, z1, y0, y1;
    axis_reach(pi.z, rcm, gi, 2, z0, z1);
    axis_reach(pi.y, rcm, gi, 1, y0, y1);
    for (int z = z0; z <= z1; ++z)
        for (int y = y0; y <= y1; ++y) {
            int x0, x1;
            if (!row_reach(pi, rcm, z, y, gi, x0, x1)) continue;
            int lo, hi;
            row_cells(gi, z, y, x0, x1, lo, hi);
            const int e = cell_start[hi + 1];
            for (int s = cell_start[lo]; s < e; ++s) {
                const float4 pj = spos[s];
                const int j = __float_as_int(pj.w);
                if (j == i) continue;
                const double d2 = pair_d2(xi, yi, zi, pj);
                if (d2 < rc2) f(j, d2);
            }
        }
}

// In-place heapsort of ints ascending.
__device__ inline void heapsort_int(int32_t *a, int len)
{
    auto sift = [&](int root, int end) {
        while (true) {
            int child = 2 * root + 1;
            if (child >= end) break;
            if (child + 1 < end && a[child + 1] > a[child]) ++child;
            if (a[root] >= a[child]) break;
            const int32_t tmp = a[root]; a[root] = a[child]; a[child] = tmp;
            root = child;
        }
    };
    for (int r = len / 2 - 1; r >= 0; --r) sift(r, len);
    for (int end = len - 1; end > 0; --end) {
        const int32_t tmp = a[0]; a[0] = a[end]; a[end] = tmp;
        sift(0, end);
    }
}

// One thread's fill of a row longer than the wave kernels' LDS buffer (kWaveCap),
// run by lane 0 of the row's wave.
__device__ __forceinline__ void fill_csr_row(int i, float4 pi, float rc, double rc2, const GridInfo &gi,
                                             const int32_t *__restrict__ cell_start,
                                             const float4 *__restrict__ spos,
                                             const int32_t *__restrict__ nbr_start, int32_t *nbr_idx)
{
    int32_t *row = nbr_idx + nbr_start[i];
    int cnt = 0;
    for_each_neighbor(i, pi, rc, rc2, gi, cell_start, spos, [&](int j, double) { row[cnt++] = j; });
    heapsort_int(row, cnt);
}

// Key order for the cap: (d2, j) lexicographic.
__device__ __forceinline__ bool key_less(double da, int ja, double db, int jb)
{
    return da < db || (da == db && ja < jb);
}

// One thread's fill of a capped row the wave kernel cannot hold or rank, run by
// lane 0 of the row's wave: a max-heap of the K nearest held in the row itself.
__device__ __forceinline__ void fill_capped_row(int i, float4 pi, int K, float rc, double rc2,
                                                const float *__restrict__ pos, const GridInfo &gi,
                                                const int32_t *__restrict__ cell_start,
                                                const float4 *__restrict__ spos, int32_t *nbr_start,
                                                int32_t *nbr_len, int32_t *nbr_idx)
{
    const double xi = pi.x, yi = pi.y, zi = pi.z;
    int32_t *row = nbr_idx + (size_t)i * K;
    // max-heap on (d2, j): row[0] is the farthest kept neighbour
    auto sift_down = [&](int root, int end) {
        int32_t rj = row[root];
        double rd = d2_of(pos, xi, yi, zi, rj);
        while (true) {
            int child = 2 * root + 1;
            if (child >= end) break;
            int32_t cj = row[child];
            double cd = d2_of(pos, xi, yi, zi, cj);
            if (child + 1 < end) {
                const int32_t c2 = row[child + 1];
                const double d2v = d2_of(pos, xi, yi, zi, c2);
                if (key_less(cd, cj, d2v, c2)) { ++child; cj = c2; cd = d2v; }
            }
            if (!key_less(rd, rj, cd, cj)) break;
            row[root] = cj;
            root = child;
        }
        row[root] = rj;
    };
    int cnt = 0;
    for_each_neighbor(i, pi, rc, rc2, gi, cell_start, spos, [&](int j, double d2) {
        if (cnt < K) {
            row[cnt] = j;
            if (cnt + 1 == K)
                for (int r = K / 2 - 1; r >= 0; --r) sift_down(r, K);
        } else {
            const int32_t tj = row[0];
            if (key_less(d2, j, d2_of(pos, xi, yi, zi, tj), tj)) {
                row[0] = j;
                sift_down(0, K);
            }
        }
        ++cnt;
    });
    const int len = cnt < K ? cnt : K;
    heapsort_int(row, len);
    for (int s = len; s < K; ++s) row[s] = -1;
    nbr_len[i] = len;
    nbr_start[i] = (int32_t)((size_t)i * K);
}

// ---------------------------------------------------------------- step 4, one wave per target
// A wave scans its target's reach 64 candidates at a time.  Cells are sorted by
// (z, y, x), so the x-cells of one (z, y) row that the sphere reaches are one
// contiguous range of the cell-sorted arrays; lane r resolves row r, and the
// rows' ranges are flattened into one candidate index space (a candidate finds
// its row by a binary search over the lanes' running totals).  Passing
// candidates are compacted into LDS (ballot + prefix count) in the scan's order
// and written out in it (no consumer needs rows sorted by j: the streaming
// kernels sort what they merge); over-cap rows are cut to the K nearest by a
// register bitonic sort of the (d2, j) keys.  Rows longer than the LDS buffer
// are filled by lane 0 alone with the per-thread code above.
constexpr int kWaveCap = 1024;                 // candidates a wave can hold in LDS
constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Decides d2 < rc2 exactly.  An fp32 estimate settles every pair whose squared
// distance is not within a relative 1e-5 of rc2 (its own error is below 4e-7
// relative: one rounding per difference, product and sum); the rest take the
// exact fp64 predicate.  The decision is therefore the fp64 one in every case.
struct CutoffTest {
    double rc2;
    float lo, hi;           // rc2 * (1 - 1e-5), rc2 * (1 + 1e-5) in fp32
    __device__ __forceinline__ CutoffTest(double r2)
        : rc2(r2), lo((float)(r2 * (1.0 - 1e-5))), hi((float)(r2 * (1.0 + 1e-5)))
    {
        if (!(lo > 1e-30f && hi < 1e30f)) {  // cutoffs outside fp32's comfortable range: always exact
            lo = -1.f;
            hi = INFINITY;
        }
    }
    __device__ __forceinline__ bool inside(double xi, double yi, double zi, float4 pi, float4 pj) const
    {
        const float dx = pj.x - pi.x, dy = pj.y - pi.y, dz = pj.z - pi.z;
        const float e = dx * dx + dy * dy + dz * dz;
        if (e < lo) return true;
        if (e > hi) return false;             // a NaN estimate falls through to the exact test
        return pair_d2(xi, yi, zi, pj) < rc2;
    }
};

// Number of neighbours of target i at position pi; with COLLECT the first kWaveCap
// of them land in cj (unordered).  Returns a wave-uniform count.  Candidate
// positions are fetched 4 x 64 at a time, so a target costs a few memory round
// trips rather than one per 64 candidates.
template <bool COLLECT>
__device__ __forceinline__ int wave_scan(int i, float4 pi, float rc, double rc2, const GridInfo &gi,
                                         const int32_t *__restrict__ cell_start, const float4 *__restrict__ spos,
                                         int32_t *cj, int lane)
{
    constexpr int U = 4;
    const double xi = pi.x, yi = pi.y, zi = pi.z;
    const CutoffTest test(rc2);
    const float rcm = rc + gi.margin;
    int z0, z1, y0, y1;
    axis_reach(pi.z, rcm, gi, 2, z0, z1);
    axis_reach(pi.y, rcm, gi, 1, y0, y1);
    const int ny = y1 - y0 + 1, nrow = (z1 - z0 + 1) * ny;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int count = 0;
    for (int rb = 0; rb < nrow; rb += 64) {           // one pass unless the reach spans > 64 rows
        // lane r: candidate range [a, a + len) of row rb + r
        int a = 0, len = 0;
        const int r = rb + lane;
        if (r < nrow) {
            const int zr = r / ny;
            const int z = z0 + zr, y = y0 + (r - zr * ny);
            int x0, x1;
            if (row_reach(pi, rcm, z, y, gi, x0, x1)) {
                int lo, hi;
                row_cells(gi, z, y, x0, x1, lo, hi);
                a = cell_start[lo];
                len = cell_start[hi + 1] - a;
            }
        }
        int incl = len;                               // running total over lanes 0..r
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const int total = __shfl(incl, 63, 64);
        const int offr = a - (incl - len);            // candidate f of row r is spos[f + offr]
        for (int c0 = 0; c0 < total; c0 += 64 * U) {
            float4 pj[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = c0 + 64 * u + lane;
                ok[u] = f < total;
                // row of f = the number of rows whose running total is <= f (totals ascend)
                int k = 0;
#pragma unroll
                for (int st = 32; st >= 1; st >>= 1) k += (__shfl(incl, k + st - 1, 64) <= f) ? st : 0;
                const int o = __shfl(offr, k, 64);
                pj[u] = ok[u] ? spos[f + o] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = __float_as_int(pj[u].w);
                const bool pass = ok[u] && j != i && test.inside(xi, yi, zi, pi, pj[u]);
                const uint64_t m = __ballot(pass);
                if (COLLECT && pass) {
                    const int slot = count + __popcll(m & below);
                    if (slot < kWaveCap) cj[slot] = j;
                }
                count += __popcll(m);
            }
        }
    }
    return count;
}

// Rows are ordered by j with wave_bitonic_sort (e2v2_internal.h).
// row[0 .. cnt) = the cnt distinct keys of cj in increasing order.
template <int E>
__device__ __forceinline__ void wave_write_sorted_n(const int32_t *cj, int cnt, int32_t *row, int lane)
{
    int a[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int e = lane * E + k;
        a[k] = e < cnt ? cj[e] : INT_MAX;
    }
    wave_bitonic_sort<E>(a, lane);
#pragma unroll
    for (int k = 0; k < E; ++k)
        if (lane * E + k < cnt) row[lane * E + k] = a[k];
}
__device__ __forceinline__ void wave_write_sorted(const int32_t *cj, int cnt, int32_t *row, int lane)
{
    if (cnt <= 64) wave_write_sorted_n<1>(cj, cnt, row, lane);
    else if (cnt <= 128) wave_write_sorted_n<2>(cj, cnt, row, lane);
    else if (cnt <= 256) wave_write_sorted_n<4>(cj, cnt, row, lane);
    else if (cnt <= 512) wave_write_sorted_n<8>(cj, cnt, row, lane);
    else wave_write_sorted_n<16>(cj, cnt, row, lane);
}

// The K nearest of cnt candidates by (d2, j), exactly: every lane computes the
// fp64 squared distances of its E candidates, the wave sorts the keys (bits of
// d2, which order like the values for d2 >= 0, then j) with a register bitonic
// sort, and cj[0 .. K) receives the first K indices (unordered by j).
constexpr int kSelectCap = 512;                 // largest candidate count ranked in registers
__device__ __forceinline__ bool key_before(uint64_t da, int ja, uint64_t db, int jb)
{
    return da < db || (da == db && ja < jb);
}
template <int E>
__device__ __forceinline__ void wave_keep_nearest_n(int32_t *cj, int cnt, int K, float4 pi, const float *__restrict__ pos,
                                                    int lane)
{
    constexpr int N = 64 * E;
    uint64_t dk[E];
    int jk[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int e = lane * E + k;
        dk[k] = ~0ull;
        jk[k] = INT_MAX;
        if (e < cnt) {
            const int j = cj[e];
            const double d2 = pair_d2((double)pi.x, (double)pi.y, (double)pi.z,
                                      make_float4(pos[3 * (size_t)j], pos[3 * (size_t)j + 1], pos[3 * (size_t)j + 2], 0.f));
            dk[k] = (uint64_t)__double_as_longlong(d2);
            jk[k] = j;
        }
    }
#pragma unroll
    for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (int d = size >> 1; d >= 1; d >>= 1) {
            if (d >= E) {
                const int lx = d / E;
                const bool asc = ((lane * E) & size) == 0;
                const bool keep_min = ((lane & lx) == 0) == asc;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const uint32_t olo = __shfl_xor((uint32_t)dk[k], lx, 64);
                    const uint32_t ohi = __shfl_xor((uint32_t)(dk[k] >> 32), lx, 64);
                    const int oj = __shfl_xor(jk[k], lx, 64);
                    const uint64_t od = ((uint64_t)ohi << 32) | olo;
                    const bool other_first = key_before(od, oj, dk[k], jk[k]);
                    if (other_first == keep_min) {
                        dk[k] = od;
                        jk[k] = oj;
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if (k & d) continue;
                    const bool asc = ((lane * E + k) & size) == 0;
                    const bool sw = asc ? key_before(dk[k | d], jk[k | d], dk[k], jk[k])
                                        : key_before(dk[k], jk[k], dk[k | d], jk[k | d]);
                    if (sw) {
                        const uint64_t td = dk[k];
                        const int tj = jk[k];
                        dk[k] = dk[k | d];
                        jk[k] = jk[k | d];
                        dk[k | d] = td;
                        jk[k | d] = tj;
                    }
                }
            }
        }
    }
    wave_lds_sync();                                  // every lane has read its candidates
#pragma unroll
    for (int k = 0; k < E; ++k)
        if (lane * E + k < K) cj[lane * E + k] = jk[k];
    wave_lds_sync();
}
__device__ __forceinline__ void wave_keep_nearest(int32_t *cj, int cnt, int K, float4 pi, const float *__restrict__ pos,
                                                  int lane)
{
    if (cnt <= 64) wave_keep_nearest_n<1>(cj, cnt, K, pi, pos, lane);
    else if (cnt <= 128) wave_keep_nearest_n<2>(cj, cnt, K, pi, pos, lane);
    else if (cnt <= 256) wave_keep_nearest_n<4>(cj, cnt, K, pi, pos, lane);
    else wave_keep_nearest_n<8>(cj, cnt, K, pi, pos, lane);
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void k_count_wave(int n, float rc, double rc2,
                                                                    const GridInfo *__restrict__ grid,
                                                                    const int32_t *__restrict__ cell_start,
                                                                    const int32_t *__restrict__ order,
                                                                    const float4 *__restrict__ spos, int32_t *nbr_len)
{
    const int lane = threadIdx.x & 63;
    const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
    if (t >= n) return;
    const GridInfo gi = *grid;
    const int i = order[t];
    const int cnt = wave_scan<false>(i, spos[t], rc, rc2, gi, cell_start, spos, nullptr, lane);
    if (lane == 0) nbr_len[i] = cnt;
}

// CSR rows; a row longer than kWaveCap entries is filled by lane 0 alone
// (fill_csr_row).
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_fill_csr_wave(int n, float rc, double rc2,
                                                                       const GridInfo *__restrict__ grid,
                                                                       const int32_t *__restrict__ cell_start,
                                                                       const int32_t *__restrict__ order,
                                                                       const float4 *__restrict__ spos,
                                                                       const int32_t *__restrict__ nbr_start,
                                                                       const int32_t *__restrict__ nbr_len, int32_t *nbr_idx)
{
    __shared__ __align__(16) int32_t sj[kWavesPerBlock][kWaveCap + 4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWavesPerBlock + w));
    if (t >= n) return;
    const int i = order[t];
    const GridInfo gi = *grid;
    if (nbr_len[i] > kWaveCap) {
        if (lane == 0) fill_csr_row(i, spos[t], rc, rc2, gi, cell_start, spos, nbr_start, nbr_idx);
        return;
    }
    const int cnt = wave_scan<true>(i, spos[t], rc, rc2, gi, cell_start, spos, sj[w], lane);
    wave_lds_sync();
    int32_t *row = nbr_idx + nbr_start[i];
    for (int e = lane; e < cnt; e += 64) row[e] = sj[w][e];     // in the scan's order
}

// Capped rows: every candidate if there are at most K, else the K nearest by
// (d2, j), in that order; written in the scan's order and padded with -1.  Rows with more than
// kSelectCap candidates over the cap, or more than kWaveCap in all, are filled by
// lane 0 alone (fill_capped_row).  Only the index buffer sits in
// LDS, so many waves share a CU.
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_fill_capped_wave(int n, int K, float rc, double rc2,
                                                                          const float *__restrict__ pos,
                                                                          const GridInfo *__restrict__ grid,
                                                                          const int32_t *__restrict__ cell_start,
                                                                          const int32_t *__restrict__ order,
                                                                          const float4 *__restrict__ spos,
                                                                          int32_t *nbr_start, int32_t *nbr_len,
                                                                          int32_t *nbr_idx)
{
    __shared__ __align__(16) int32_t sj[kWavesPerBlock][kWaveCap + 4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWavesPerBlock + w));
    if (t >= n) return;
    const int i = order[t];
    const GridInfo gi = *grid;
    int32_t *cj = sj[w];
    const float4 pi = spos[t];
    const int cnt = wave_scan<true>(i, pi, rc, rc2, gi, cell_start, spos, cj, lane);
    int32_t *row = nbr_idx + (size_t)i * K;
    if (lane == 0) nbr_start[i] = (int32_t)((size_t)i * K);
    if (cnt > kWaveCap || (cnt > K && cnt > kSelectCap)) {
        if (lane == 0) fill_capped_row(i, pi, K, rc, rc2, pos, gi, cell_start, spos, nbr_start, nbr_len, nbr_idx);
        return;
    }
    wave_lds_sync();
    int len = cnt;
    if (cnt > K) {
        wave_keep_nearest(cj, cnt, K, pi, pos, lane);
        len = K;
    }
    for (int e = lane; e < len; e += 64) row[e] = cj[e];         // in the scan's (or the cut's) order
    for (int sidx = len + lane; sidx < K; sidx += 64) row[sidx] = -1;
    if (lane == 0) nbr_len[i] = len;
}

// ---------------------------------------------------------------- list maintenance
// Between rebuilds a model reuses the topology (Tessera article, neighbour reuse):
// lists at smaller cutoffs are the entries of the largest-cutoff list that pass
// the same fp64 predicate, and the rebuild rule needs the largest displacement
// since the last rebuild.
constexpr int kFilterWaves = 4;

// One wave per row: entries j in [0, n) with d2 < rc2, kept in order (ballot
// compaction), the rest of the row's range set to -1.  A kept entry moves only to
// an earlier slot of its row, after its chunk has been read, so out may alias in.
__global__ __launch_bounds__(64 * kFilterWaves) void k_filter_rows(const float *__restrict__ pos, int n, double rc2,
                                                                   const int32_t *start, const int32_t *len,
                                                                   const int32_t *idx, int32_t *out_len,
                                                                   int32_t *out_idx)
{
    const int lane = threadIdx.x & 63;
    const long long i = (long long)blockIdx.x * kFilterWaves + (threadIdx.x >> 6);
    if (i >= n) return;
    const long long s0 = start[i];
    const int L = len[i] > 0 ? len[i] : 0;
    const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
    int kept = 0;
    for (int base = 0; base < L; base += 64) {
        const int x = base + lane;
        int j = -1;
        bool keep = false;
        if (x < L) {
            j = idx[s0 + x];
            if (j >= 0 && j < n) keep = d2_of(pos, xi, yi, zi, j) < rc2;
        }
        const unsigned long long m = __builtin_amdgcn_ballot_w64(keep);
        const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        if (keep) out_idx[s0 + kept + before] = j;
        kept += __popcll(m);
    }
    for (int x = kept + lane; x < L; x += 64) out_idx[s0 + x] = -1;
    if (lane == 0) out_len[i] = kept;
}

// Largest (dx*dx + dy*dy) + dz*dz over atoms, fp64 (dx = x - x_ref of fp32 values is
// exact), a non-finite value counting as +inf; *out must hold 0 beforehand.  The
// bit patterns of non-negative doubles order like their values, so blocks combine
// with an integer atomic max.
__global__ __launch_bounds__(256) void k_max_disp2(const float *__restrict__ pos, const float *__restrict__ ref, int n,
                                                   unsigned long long *out)
{
    __shared__ double sm[4];
    double m = 0.0;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
        const double dx = (double)pos[3 * i] - (double)ref[3 * i];
        const double dy = (double)pos[3 * i + 1] - (double)ref[3 * i + 1];
        const double dz = (double)pos[3 * i + 2] - (double)ref[3 * i + 2];
        const double xx = dx * dx, yy = dy * dy, zz = dz * dz;
        double d2 = (xx + yy) + zz;
        if (!(d2 <= 1.7976931348623157e308)) d2 = INFINITY;   // NaN and inf
        m = d2 > m ? d2 : m;
    }
    for (int o = 32; o > 0; o >>= 1) {
        const double v = __shfl_xor(m, o, 64);
        m = v > m ? v : m;
    }
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) m = sm[w] > m ? sm[w] : m;
        atomicMax(out, (unsigned long long)__double_as_longlong(m));
    }
}

// ---------------------------------------------------------------- host launchers
// ---------------------------------------------------------------- transposed list
// The sources' view of a neighbour list: row j of the transposed list holds every
// i whose row contains j (an entry listed twice appears twice), in increasing
// order, so sums over it run in a fixed order.  Entries < 0 or >= n are skipped,
// as the layer skips them.  Built by count, scan, fill, then a sort per row.
__global__ void k_tzero(int32_t *cnt, int n)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t <= n) cnt[t] = 0;
}
__global__ __launch_bounds__(256) void k_tcount(const int32_t *__restrict__ start, const int32_t *__restrict__ len,
                                                const int32_t *__restrict__ idx, int n, int32_t *cnt)
{
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (i >= n) return;
    const int s0 = start[i], l = len[i];
    for (int p = lane; p < l; p += 64) {
        const int j = idx[s0 + p];
        if (j >= 0 && j < n) atomicAdd(&cnt[j], 1);
    }
}
__global__ __launch_bounds__(256) void k_tfill(const int32_t *__restrict__ start, const int32_t *__restrict__ len,
                                               const int32_t *__restrict__ idx, int n, long long cap, int32_t *cur,
                                               int32_t *tidx)
{
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (i >= n) return;
    const int s0 = start[i], l = len[i];
    for (int p = lane; p < l; p += 64) {
        const int j = idx[s0 + p];
        if (j < 0 || j >= n) continue;
        const int slot = atomicAdd(&cur[j], 1);
        if (slot < cap) tidx[slot] = i;
    }
}
// One 64-lane block per row: a register bitonic sort up to 1024 entries, an
// odd-even transposition sort in place beyond.
__global__ __launch_bounds__(64) void k_tsort(const int32_t *__restrict__ tstart, int n, long long cap, int32_t *tidx,
                                              int32_t *tlen)
{
    const int j = blockIdx.x, lane = threadIdx.x;
    const long long a = tstart[j], b0 = tstart[j + 1];
    const long long b = b0 < cap ? b0 : cap;
    const int cnt = b > a ? (int)(b - a) : 0;
    int32_t *row = tidx + a;
    if (lane == 0) tlen[j] = cnt;
    if (cnt <= 1) return;
    if (cnt <= 1024) {
        wave_write_sorted(row, cnt, row, lane);
        return;
    }
    for (int ph = 0; ph < cnt; ++ph) {
        for (int q = 2 * lane + (ph & 1); q + 1 < cnt; q += 128) {
            const int x = row[q], y = row[q + 1];
            if (x > y) { row[q] = y; row[q + 1] = x; }
        }
        __syncthreads();
    }
}

hipError_t launch_transpose_list(const int32_t *start, const int32_t *len, const int32_t *idx, int n,
                                 long long cap, int32_t *cnt, int32_t *tstart, int32_t *cur, int32_t *tidx,
                                 int32_t *tlen, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    k_tzero<<<(unsigned)((n + 256) / 256), 256, 0, stream>>>(cnt, n);
    const unsigned g4 = (unsigned)((n + 3) / 4);
    k_tcount<<<g4, 256, 0, stream>>>(start, len, idx, n, cnt);
    k_scan<<<1, 1024, 0, stream>>>(cnt, nullptr, n, tstart, cur, nullptr);
    k_tfill<<<g4, 256, 0, stream>>>(start, len, idx, n, cap, cur, tidx);
    k_tsort<<<(unsigned)n, 64, 0, stream>>>(tstart, n, cap, tidx, tlen);
    return hipGetLastError();
}

static inline unsigned nblk(long long n, int b) { return (unsigned)((n + b - 1) / b); }

hipError_t launch_filter_rows(const float *pos, int n, float cutoff, const int32_t *start, const int32_t *len,
                              const int32_t *idx, int32_t *out_len, int32_t *out_idx, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const double rc2 = (double)cutoff * (double)cutoff;
    k_filter_rows<<<nblk(n, kFilterWaves), 64 * kFilterWaves, 0, stream>>>(pos, n, rc2, start, len, idx, out_len,
                                                                           out_idx);
    return hipGetLastError();
}

hipError_t launch_max_disp2(const float *pos, const float *ref, int n, double *out, hipStream_t stream)
{
    hipError_t e = hipMemsetAsync(out, 0, sizeof(double), stream);
    if (e != hipSuccess || n <= 0) return e;
    const unsigned nb = (unsigned)std::min<long long>(1024, ((long long)n + 255) / 256);
    k_max_disp2<<<nb, 256, 0, stream>>>(pos, ref, n, reinterpret_cast<unsigned long long *>(out));
    return hipGetLastError();
}

hipError_t launch_neighbors_count(const float *pos, int n, float cutoff, int K, void *ws, size_t,
                                  int32_t *nbr_len, int32_t *order_out, hipStream_t stream)
{
    NbrLayout L = nbr_layout(ws, n);
    const int maxc = max_cells(n);
    const int nparts = (int)std::min<long long>(kBoxBlocks, ((long long)n + 255) / 256);
    // with order_out the Hilbert processing order (curve.h) rides along in the same
    // launches: its box, indices and bucket counts, bucket scan, slots and ranks
    const bool ord = order_out != nullptr;
    curve::CurveInfo *ci = ord ? L.curve : nullptr;
    k_bbox_partial<<<nparts, 256, 0, stream>>>(pos, n, L.box_part, maxc, L.cell_cnt, ord ? L.bcnt : nullptr);
    k_cell_assign<<<nblk(n, 256), 256, 0, stream>>>(pos, n, L.box_part, nparts, cutoff, maxc, L.grid, L.cell_of,
                                                    L.cell_cnt, ci, L.key, L.bcnt);
    if (ord)
        k_scan_cells_buckets<<<2, kScanThreads, 0, stream>>>(L.cell_cnt, &L.grid->ncell, L.cell_start, L.cell_cur, L.bcnt,
                                                     L.bstart, L.bcursor, L.items, L.nitems);
    else
        k_scan<<<1, 1024, 0, stream>>>(L.cell_cnt, &L.grid->ncell, 0, L.cell_start, L.cell_cur, nullptr);
    k_scatter<<<nblk(n, 256), 256, 0, stream>>>(n, L.cell_of, L.cell_cur, L.mval, ci, L.key, L.bcursor, L.ent);
    const unsigned nplace = nblk(n, 256);
    const unsigned nrank = ord ? nblk(curve::max_items(n), 4) : 0u;
    k_place<<<nplace + nrank, 256, 0, stream>>>(pos, n, L.cell_of, L.cell_start, L.mval, L.order, L.spos, nplace,
                                                L.ent, L.bstart, L.items, L.nitems, order_out);
    if (K == 0) {
        const double rc2 = (double)cutoff * (double)cutoff;
        k_count_wave<<<nblk(n, kWavesPerBlock), 64 * kWavesPerBlock, 0, stream>>>(n, cutoff, rc2, L.grid, L.cell_start,
                                                                                L.order, L.spos, nbr_len);
    }
    return hipGetLastError();
}

hipError_t launch_neighbors_scan(int n, void *ws, int32_t *nbr_start, int32_t *nbr_len, int64_t *nnz_dev,
                                 hipStream_t stream)
{
    // nbr_start needs n + 1 slots for the scan's total; use the layout's cell_start
    // scratch for the tail-inclusive copy and write the first n into nbr_start.
    NbrLayout L = nbr_layout(ws, n);
    k_scan<<<1, 1024, 0, stream>>>(nbr_len, nullptr, n, L.cell_cur, nbr_start, nnz_dev);
    return hipGetLastError();
}

hipError_t launch_neighbors_fill(const float *pos, int n, float cutoff, int K, void *ws, int32_t *nbr_start,
                                 int32_t *nbr_len, int32_t *nbr_idx, hipStream_t stream)
{
    NbrLayout L = nbr_layout(ws, n);
    const double rc2 = (double)cutoff * (double)cutoff;
    if (K == 0) {
        k_fill_csr_wave<<<nblk(n, kWavesPerBlock), 64 * kWavesPerBlock, 0, stream>>>(
            n, cutoff, rc2, L.grid, L.cell_start, L.order, L.spos, nbr_start, nbr_len, nbr_idx);
    } else {
        k_fill_capped_wave<<<nblk(n, kWavesPerBlock), 64 * kWavesPerBlock, 0, stream>>>(
            n, K, cutoff, rc2, pos, L.grid, L.cell_start, L.order, L.spos, nbr_start, nbr_len, nbr_idx);
    }
    return hipGetLastError();
}

}  // namespace e2v2
