// Per-node linear projections on the matrix cores: q = h^0 W_Q, k = h^0 W_K,
// v^l = h^l W_V[l] and out^l = hhat^l W_O[l] -- the layer's only dense
// contractions.  Each (component, weight) pair is one "job"; rows of a job are
// nodes.  One wave computes a 16-node x C tile with v_mfma_f32_16x16x4_f32
// (fp32 accumulate; bf16 operands are widened exactly on load).
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
