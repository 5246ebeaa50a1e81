// Per-node linear projections for fp32 storage, and the packing of bf16 weights
// for the 16-bit path.  The projections q = h^0 W_Q, k = h^0 W_K, v^l = h^l W_V[l]
// and out^l = hhat^l W_O[l] are the layer's only dense contractions (E2Former-V2
// explainer, section 5.1: projections around the equivariant core).
//
// fp32 storage: each (component, weight) pair is one "job" whose rows are nodes,
// on v_mfma_f32_16x16x4_f32 with one wave per 16-node x C tile.  The contraction
// index is permuted so that each lane's 16 x 4 A fragment comes from one
// contiguous stretch of its row: in MFMA step s, lane group g (lanes 16g..16g+15)
// supplies k = g*C/4 + s for both A and B.  Any bijection of k gives the same sum;
// this one turns the A loads into 16-byte vectors.
//
// 16-bit storage runs the projections fused with the couplings (qkv_eaas.hip,
// eaas_outproj.hip) on v_mfma_f32_16x16x32_bf16; k_pack_wt below lays the bf16
// weights out as that instruction's A fragments.
#include "e2v2_internal.h"

#include <algorithm>

namespace e2v2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMaxJobs = 18;
struct ProjJobs {
    ProjJob j[kMaxJobs];
};

// KQ = C / 4 contraction indices per lane group.  A wave covers RT tiles of 16
// rows, so each B value it loads feeds RT matrix-core steps; launches with few
// jobs take RT = 1 to keep enough waves in flight.
template <int KQ, int RT>
__global__ __launch_bounds__(64) void proj_kernel(const ProjJobs jobs, int n)
{
    constexpr int C = 4 * KQ;
    const ProjJob &job = jobs.j[blockIdx.y];
    const int lane = threadIdx.x;
    const int g = lane >> 4, m = lane & 15;
    const long long row0 = (long long)blockIdx.x * (16 * RT);
    float a[RT][KQ];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const long long row = row0 + rt * 16 + m;
        if (row < n) {
            const float *ap = reinterpret_cast<const float *>(job.a) + row * job.a_node_stride + (long long)job.comp * C + g * KQ;
#pragma unroll
            for (int e = 0; e < KQ; e += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(ap + e);
                a[rt][e] = v.x; a[rt][e + 1] = v.y; a[rt][e + 2] = v.z; a[rt][e + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < KQ; ++e) a[rt][e] = 0.f;
        }
    }
    for (int nb = 0; nb < C / 16; ++nb) {
        // B element (k, n) for k = g KQ + s, n = 16 nb + m: b[k][n], or b[n][k] for the
        // transposed weight (one contiguous stretch of a row, read as 16-byte vectors)
        float bb[KQ];
        if (job.b_trans) {
            const float *bt = reinterpret_cast<const float *>(job.b) + (long long)(nb * 16 + m) * C + g * KQ;
#pragma unroll
            for (int e = 0; e < KQ; e += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(bt + e);
                bb[e] = v.x; bb[e + 1] = v.y; bb[e + 2] = v.z; bb[e + 3] = v.w;
            }
        } else {
            const float *bp = reinterpret_cast<const float *>(job.b) + (long long)(g * KQ) * C + nb * 16 + m;
#pragma unroll
            for (int e = 0; e < KQ; ++e) bb[e] = bp[(long long)e * C];
        }
        floatx4 acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KQ; ++s2)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt][s2], bb[s2], acc[rt], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const long long orow = row0 + rt * 16 + 4 * g + r;
                if (orow < n) {
                    float *o = job.out + orow * job.o_node_stride + (long long)job.comp * C + nb * 16 + m;
                    *o = job.accumulate ? *o + acc[rt][r] : acc[rt][r];
                }
            }
    }
}

// ---------------------------------------------------------------------------
// bf16 weights as A fragments of v_mfma_f32_16x16x32_bf16 in the transposed
// orientation out^T = W^T . in^T: a wave reads one 16 x 32 fragment of W^T as one
// coalesced 1 KB load.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// W [C][C] (in, out) bf16 -> fragments: for output block nb (16 channels) and
// contraction block kb (32 indices), lane l holds W[32 kb + 8 (l / 16) + e][16 nb + l % 16], e < 8.
constexpr int kMaxPack = 64;          // matrices per packing launch (a whole layer stack)
struct PackJobs {
    const uint16_t *w[kMaxPack];
    uint16_t *out[kMaxPack];
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

hipError_t launch_pack_weights(const uint16_t *const *w, uint16_t *const *out, int count, int C, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    if (count > kMaxPack || C % 32 != 0) return hipErrorInvalidValue;
    PackJobs pj{};
    for (int i = 0; i < count; ++i) {
        pj.w[i] = w[i];
        pj.out[i] = out[i];
    }
    const int threads = (C / 16) * (C / 32) * 64;
    k_pack_wt<<<dim3((unsigned)((threads + 255) / 256), (unsigned)count), 256, 0, stream>>>(pj, C);
    return hipGetLastError();
}

// bf16 -> fp32 (exact), 8 values per thread where the count allows, grid-stride.
__global__ __launch_bounds__(256) void k_widen_bf16(const uint16_t *__restrict__ in, float *__restrict__ out, long long count)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    const long long n8 = count >> 3;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
        const uint4 v = reinterpret_cast<const uint4 *>(in)[i];
        float4 *o = reinterpret_cast<float4 *>(out) + 2 * i;
        o[0] = make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
        o[1] = make_float4(bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w));
    }
    for (long long i = 8 * n8 + (long long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        out[i] = bf16_to_f(in[i]);
}

hipError_t launch_widen_bf16(const void *in, float *out, long long count, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    long long blocks = ((count >> 3) + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    k_widen_bf16<<<dim3((unsigned)blocks), 256, 0, stream>>>(reinterpret_cast<const uint16_t *>(in), out, count);
    return hipGetLastError();
}

hipError_t launch_proj(const ProjJob *jobs, int njobs, int n, int C, hipStream_t stream)
{
    if (n <= 0 || njobs <= 0) return hipSuccess;
    if (njobs > kMaxJobs) return hipErrorInvalidValue;
    ProjJobs pj{};
    for (int i = 0; i < njobs; ++i) pj.j[i] = jobs[i];
    const int rt = njobs >= 4 ? 4 : 1;
    dim3 grid((unsigned)((n + 16 * rt - 1) / (16 * rt)), (unsigned)njobs), block(64);
    switch (C * 8 + rt) {
    case 32 * 8 + 1: proj_kernel<8, 1><<<grid, block, 0, stream>>>(pj, n); break;
    case 32 * 8 + 4: proj_kernel<8, 4><<<grid, block, 0, stream>>>(pj, n); break;
    case 64 * 8 + 1: proj_kernel<16, 1><<<grid, block, 0, stream>>>(pj, n); break;
    case 64 * 8 + 4: proj_kernel<16, 4><<<grid, block, 0, stream>>>(pj, n); break;
    case 128 * 8 + 1: proj_kernel<32, 1><<<grid, block, 0, stream>>>(pj, n); break;
    case 128 * 8 + 4: proj_kernel<32, 4><<<grid, block, 0, stream>>>(pj, n); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace e2v2
