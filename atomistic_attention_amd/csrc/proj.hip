// Per-node linear projections on the matrix cores: q = h^0 W_Q, k = h^0 W_K,
// v^l = h^l W_V[l] and out^l = hhat^l W_O[l] -- the layer's only dense
// contractions.  Each (component, weight) pair is one "job"; rows of a job are
// nodes.  bf16 weights use the bf16 kernel below; fp32 weights use
// v_mfma_f32_16x16x4_f32 with one wave per 16-node x C tile.
//
// The contraction index is permuted so that each lane's 16 x 4 A fragment
// comes from one contiguous stretch of its row: in MFMA step s, lane group g
// (lanes 16g..16g+15) supplies k = g*C/4 + s for both A and B.  Any bijection
// of k gives the same sum; this one turns the A loads into 16-byte vectors.
#include "e2v2_internal.h"

namespace e2v2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMaxJobs = 18;
struct ProjJobs {
    ProjJob j[kMaxJobs];
};

template <typename TA> __device__ __forceinline__ void load_row(const TA *p, int cnt, float *dst);
template <> __device__ __forceinline__ void load_row<float>(const float *p, int cnt, float *dst)
{
    for (int e = 0; e < cnt; e += 4) {
        float4 v = *reinterpret_cast<const float4 *>(p + e);
        dst[e] = v.x; dst[e + 1] = v.y; dst[e + 2] = v.z; dst[e + 3] = v.w;
    }
}
template <> __device__ __forceinline__ void load_row<uint16_t>(const uint16_t *p, int cnt, float *dst)
{
    for (int e = 0; e < cnt; e += 8) {
        uint4 v = *reinterpret_cast<const uint4 *>(p + e);
        dst[e + 0] = bf16lo(v.x); dst[e + 1] = bf16hi(v.x);
        dst[e + 2] = bf16lo(v.y); dst[e + 3] = bf16hi(v.y);
        dst[e + 4] = bf16lo(v.z); dst[e + 5] = bf16hi(v.z);
        dst[e + 6] = bf16lo(v.w); dst[e + 7] = bf16hi(v.w);
    }
}
template <typename TB> __device__ __forceinline__ float ld_w(const TB *p);
template <> __device__ __forceinline__ float ld_w<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld_w<uint16_t>(const uint16_t *p) { return bf16_to_f(*p); }

// KQ = C / 4 contraction indices per lane group.
template <typename TA, typename TB, int KQ>
__global__ __launch_bounds__(64) void proj_kernel(const ProjJobs jobs, int n)
{
    constexpr int C = 4 * KQ;
    const ProjJob &job = jobs.j[blockIdx.y];
    const int lane = threadIdx.x;
    const int g = lane >> 4, m = lane & 15;
    const long long row = (long long)blockIdx.x * 16 + m;
    float a[KQ];
    if (row < n) {
        const TA *ap = reinterpret_cast<const TA *>(job.a) + row * job.a_node_stride + (long long)job.comp * C + g * KQ;
        load_row<TA>(ap, KQ, a);
    } else {
#pragma unroll
        for (int e = 0; e < KQ; ++e) a[e] = 0.f;
    }
    const TB *bp = reinterpret_cast<const TB *>(job.b) + (long long)(g * KQ) * C + m;
    const long long orow0 = (long long)blockIdx.x * 16 + 4 * g;
    for (int nb = 0; nb < C / 16; ++nb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KQ; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], ld_w<TB>(bp + (long long)s * C + nb * 16), acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const long long orow = orow0 + r;
            if (orow < n) job.out[orow * job.o_node_stride + (long long)job.comp * C + nb * 16 + m] = acc[r];
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 path on v_mfma_f32_16x16x32_bf16, in the transposed orientation
// out^T = W^T . in^T: the 16 x 32 A operand is a fragment of W^T, pre-packed so a
// wave reads it as one coalesced 1 KB load; the 32 x 16 B operand is 16 nodes'
// input rows (8 consecutive contraction indices per lane, one 16-byte load);
// each lane of the 16 x 16 result holds 4 consecutive output channels of one
// node and writes them as one 16-byte store.  fp32 inputs (hhat) are split into
// bf16 hi + lo, two products, which keeps about 16 significant bits of the
// input against exact bf16 weights.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// W [C][C] (in, out) bf16 -> fragments: for output block nb (16 channels) and
// contraction block kb (32 indices), lane l holds W[32 kb + 8 (l / 16) + e][16 nb + l % 16], e < 8.
struct PackJobs {
    const uint16_t *w[kMaxJobs];
    uint16_t *out[kMaxJobs];
};
__global__ void k_pack_wt(const PackJobs pj, int C)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int KB = C / 32, NB = C / 16;
    if (t >= NB * KB * 64) return;
    const int lane = t & 63, frag = t >> 6, nb = frag / KB, kb = frag - nb * KB;
    const int nn = 16 * nb + (lane & 15), k0 = 32 * kb + 8 * (lane >> 4);
    const uint16_t *w = pj.w[blockIdx.y];
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = w[(size_t)(k0 + e) * C + nn];
    uint4 o;
    o.x = v[0] | (uint32_t(v[1]) << 16);
    o.y = v[2] | (uint32_t(v[3]) << 16);
    o.z = v[4] | (uint32_t(v[5]) << 16);
    o.w = v[6] | (uint32_t(v[7]) << 16);
    reinterpret_cast<uint4 *>(pj.out[blockIdx.y])[t] = o;
}

template <bool AF32, int C>
__global__ __launch_bounds__(256) void proj_bf16_kernel(const ProjJobs jobs, int n)
{
    constexpr int KB = C / 32, NB = C / 16;
    const ProjJob &job = jobs.j[blockIdx.y];
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long node = tile * 16 + (lane & 15);
    const bool valid = node < n;
    bf16x8 bhi[KB], blo[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        uint4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
        if (valid) {
            if constexpr (AF32) {
                const float *ap = reinterpret_cast<const float *>(job.a) + node * job.a_node_stride +
                                  (long long)job.comp * C + 32 * kb + 8 * g;
                const float4 x0 = reinterpret_cast<const float4 *>(ap)[0];
                const float4 x1 = reinterpret_cast<const float4 *>(ap)[1];
                const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                uint16_t h16[8], l16[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    h16[e] = f_to_bf16(xs[e]);
                    l16[e] = f_to_bf16(xs[e] - bf16_to_f(h16[e]));
                }
                hi = make_uint4(h16[0] | (uint32_t(h16[1]) << 16), h16[2] | (uint32_t(h16[3]) << 16),
                                h16[4] | (uint32_t(h16[5]) << 16), h16[6] | (uint32_t(h16[7]) << 16));
                lo = make_uint4(l16[0] | (uint32_t(l16[1]) << 16), l16[2] | (uint32_t(l16[3]) << 16),
                                l16[4] | (uint32_t(l16[5]) << 16), l16[6] | (uint32_t(l16[7]) << 16));
            } else {
                hi = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(job.a) +
                                                      node * job.a_node_stride + (long long)job.comp * C +
                                                      32 * kb + 8 * g);
            }
        }
        bhi[kb] = __builtin_bit_cast(bf16x8, hi);
        blo[kb] = __builtin_bit_cast(bf16x8, lo);
    }
    const uint4 *wp = reinterpret_cast<const uint4 *>(job.b);
    float *op = job.out + node * job.o_node_stride + (long long)job.comp * C + 4 * g;
#pragma unroll 2
    for (int nb = 0; nb < NB; ++nb) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 wf = __builtin_bit_cast(bf16x8, wp[(nb * KB + kb) * 64 + lane]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, bhi[kb], acc, 0, 0, 0);
            if constexpr (AF32) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, blo[kb], acc, 0, 0, 0);
        }
        if (valid) *reinterpret_cast<float4 *>(op + 16 * nb) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

// ---------------------------------------------------------------------------
// Output projection out^l = hhat^l W_O[l] for fp32 hhat and packed bf16 weights,
// weight-stationary and persistent: a block owns one degree l, keeps its waves'
// W_O[l] fragments in registers for its whole run and streams tiles (16 nodes x
// one component of degree l) through a double-buffered LDS copy of the input
// rows, split once into bf16 hi + lo.  Tile loads run two tiles ahead.
template <int C>
__global__ __launch_bounds__(64 * (C >= 64 ? 4 : 2)) void outproj_kernel(const OutProjArgs a)
{
    constexpr int NW = C >= 64 ? 4 : 2;            // waves per block
    constexpr int NB = C / 16, KB = C / 32, NBW = NB / NW;
    constexpr int NT = 64 * NW;
    constexpr int UNITS = 2 * C;                   // 8-float units per tile (16 rows x C / 8)
    constexpr int UPT = (UNITS + NT - 1) / NT;
    constexpr int RS = C * 2 + 16;                 // LDS bytes per bf16 row (pad spreads banks)
    __shared__ __align__(16) unsigned char sA[2][2][16 * RS];   // [buffer][hi, lo][row]

    int l = 0;
    while (l < a.lmax && (int)blockIdx.x >= a.blk_start[l + 1]) ++l;
    const int nm = 2 * l + 1, NC = (a.lmax + 1) * (a.lmax + 1);
    const long long tiles = (long long)((a.n + 15) / 16) * nm;
    const long long tbase = (long long)(blockIdx.x - a.blk_start[l]) * a.tpb;
    const int cnt = (int)((tiles - tbase) < a.tpb ? (tiles - tbase) : a.tpb);
    if (cnt <= 0) return;

    const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, nl = lane & 15;
    bf16x8 wf[NBW][KB];
    const uint4 *wl = a.wo + (size_t)l * (C * C / 8);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) wf[j][kb] = __builtin_bit_cast(bf16x8, wl[((w * NBW + j) * KB + kb) * 64 + lane]);

    // tile index -> first input/output element of its rows: node 16 gi + r, component l^2 + m
    auto tile_row = [&](int it, int r, bool &ok) -> long long {
        const long long ti = tbase + it;
        const long long gi = ti / nm;
        const int m = (int)(ti - gi * nm);
        const long long node = gi * 16 + r;
        ok = node < a.n;
        return (node * NC + l * l + m) * C;
    };
    typedef float4 Stage[UPT][2];
    auto load = [&](int it, Stage &rg) {
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int u = t + j * NT;
            rg[j][0] = rg[j][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u < UNITS) {
                const int r = u / (C / 8), kc = u - r * (C / 8);
                bool ok;
                const long long o = tile_row(it, r, ok);
                if (ok) {
                    const float4 *src = reinterpret_cast<const float4 *>(a.hhat + o + 8 * kc);
                    rg[j][0] = src[0];
                    rg[j][1] = src[1];
                }
            }
        }
    };
    auto stage = [&](int buf, const Stage &rg) {
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int u = t + j * NT;
            if (u < UNITS) {
                const int r = u / (C / 8), kc = u - r * (C / 8);
                const float xs[8] = {rg[j][0].x, rg[j][0].y, rg[j][0].z, rg[j][0].w,
                                     rg[j][1].x, rg[j][1].y, rg[j][1].z, rg[j][1].w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint16_t h0 = f_to_bf16(xs[2 * e]), h1 = f_to_bf16(xs[2 * e + 1]);
                    const uint16_t l0 = f_to_bf16(xs[2 * e] - bf16_to_f(h0));
                    const uint16_t l1 = f_to_bf16(xs[2 * e + 1] - bf16_to_f(h1));
                    hi[e] = h0 | (uint32_t(h1) << 16);
                    lo[e] = l0 | (uint32_t(l1) << 16);
                }
                *reinterpret_cast<uint4 *>(&sA[buf][0][r * RS + kc * 16]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                *reinterpret_cast<uint4 *>(&sA[buf][1][r * RS + kc * 16]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
        }
    };
    auto compute = [&](int it, int buf) {
        floatx4 acc[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int off = nl * RS + kb * 64 + g * 16;
            const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&sA[buf][0][off]));
            const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&sA[buf][1][off]));
#pragma unroll
            for (int j = 0; j < NBW; ++j) {
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j][kb], bh, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j][kb], bl, acc[j], 0, 0, 0);
            }
        }
        bool ok;
        const long long o = tile_row(it, nl, ok);
        if (ok) {
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                *reinterpret_cast<float4 *>(a.out + o + 16 * (w * NBW + j) + 4 * g) =
                    make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        }
    };

    Stage p0, p1;
    load(0, p0);
    if (cnt > 1) load(1, p1);
    stage(0, p0);
    __syncthreads();
    for (int it = 0; it < cnt; it += 2) {
        // p1 holds tile it + 1; p0 is free
        if (it + 2 < cnt) load(it + 2, p0);
        compute(it, 0);
        if (it + 1 < cnt) stage(1, p1);
        __syncthreads();
        if (it + 1 >= cnt) break;
        // p0 holds tile it + 2; p1 is free
        if (it + 3 < cnt) load(it + 3, p1);
        compute(it + 1, 1);
        if (it + 2 < cnt) stage(0, p0);
        __syncthreads();
    }
}

hipError_t launch_outproj_bf16(const OutProjArgs &in, int C, hipStream_t stream)
{
    if (in.n <= 0) return hipSuccess;
    if (in.lmax < 0 || in.lmax > kMaxL) return hipErrorInvalidValue;
    OutProjArgs a = in;
    const long long groups = (a.n + 15) / 16, total = groups * (a.lmax + 1) * (a.lmax + 1);
    const long long target = 2048;                           // about eight blocks per CU
    a.tpb = (int)((total + target - 1) / target);
    a.blk_start[0] = 0;
    for (int l = 0; l <= a.lmax; ++l) {
        const long long tl = groups * (2 * l + 1);
        a.blk_start[l + 1] = a.blk_start[l] + (int)((tl + a.tpb - 1) / a.tpb);
    }
    const dim3 grid((unsigned)a.blk_start[a.lmax + 1]);
    switch (C) {
    case 32: outproj_kernel<32><<<grid, 128, 0, stream>>>(a); break;
    case 64: outproj_kernel<64><<<grid, 256, 0, stream>>>(a); break;
    case 128: outproj_kernel<128><<<grid, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pack_weights(const uint16_t *const *w, uint16_t *const *out, int count, int C, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    if (count > kMaxJobs || C % 32 != 0) return hipErrorInvalidValue;
    PackJobs pj{};
    for (int i = 0; i < count; ++i) {
        pj.w[i] = w[i];
        pj.out[i] = out[i];
    }
    const int threads = (C / 16) * (C / 32) * 64;
    k_pack_wt<<<dim3((unsigned)((threads + 255) / 256), (unsigned)count), 256, 0, stream>>>(pj, C);
    return hipGetLastError();
}

hipError_t launch_proj_bf16(const ProjJob *jobs, int njobs, int a_f32, int n, int C, hipStream_t stream)
{
    if (n <= 0 || njobs <= 0) return hipSuccess;
    if (njobs > kMaxJobs) return hipErrorInvalidValue;
    ProjJobs pj{};
    for (int i = 0; i < njobs; ++i) pj.j[i] = jobs[i];
    dim3 grid((unsigned)((n + 63) / 64), (unsigned)njobs), block(256);
#define E2V2_PROJ_BF16(CC)                                                                         \
    (a_f32 ? (proj_bf16_kernel<true, CC><<<grid, block, 0, stream>>>(pj, n), 0)                   \
           : (proj_bf16_kernel<false, CC><<<grid, block, 0, stream>>>(pj, n), 0))
    switch (C) {
    case 32: E2V2_PROJ_BF16(32); break;
    case 64: E2V2_PROJ_BF16(64); break;
    case 128: E2V2_PROJ_BF16(128); break;
    default: return hipErrorInvalidValue;
    }
#undef E2V2_PROJ_BF16
    return hipGetLastError();
}

template <typename TA, typename TB>
static hipError_t launch_proj_t(const ProjJobs &jobs, int njobs, int n, int C, hipStream_t stream)
{
    dim3 grid((unsigned)((n + 15) / 16), (unsigned)njobs), block(64);
    switch (C) {
    case 32: proj_kernel<TA, TB, 8><<<grid, block, 0, stream>>>(jobs, n); break;
    case 64: proj_kernel<TA, TB, 16><<<grid, block, 0, stream>>>(jobs, n); break;
    case 128: proj_kernel<TA, TB, 32><<<grid, block, 0, stream>>>(jobs, n); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_proj(const ProjJob *jobs, int njobs, int a_bf16, int b_bf16, int n, int C, hipStream_t stream)
{
    if (n <= 0 || njobs <= 0) return hipSuccess;
    if (njobs > kMaxJobs) return hipErrorInvalidValue;
    ProjJobs pj{};
    for (int i = 0; i < njobs; ++i) pj.j[i] = jobs[i];
    if (a_bf16 && b_bf16) return launch_proj_t<uint16_t, uint16_t>(pj, njobs, n, C, stream);
    if (a_bf16) return launch_proj_t<uint16_t, float>(pj, njobs, n, C, stream);
    if (b_bf16) return launch_proj_t<float, uint16_t>(pj, njobs, n, C, stream);
    return launch_proj_t<float, float>(pj, njobs, n, C, stream);
}

}  // namespace e2v2
