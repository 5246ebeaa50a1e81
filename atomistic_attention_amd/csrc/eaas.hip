// EAAS tensor product of node features with the encoding of the node's own
// position (E2Former-V2 explainer, section 2.1 pseudocode: alignment rotation,
// rotate features, sparse re-index, inverse rotation; section 2.3 Proposition
// 4.3: the result equals the dense SO(3) tensor product).
//
// Each node's Wigner-D blocks are built once in fp64 and shared through LDS;
// each (node, channel) pair then applies rotate-in, the m re-index and
// rotate-out entirely in registers.  Reads and writes are channel-contiguous.
#include "e2v2_internal.h"

namespace e2v2 {

template <typename T> __device__ __forceinline__ float ld_elem(const T *p, size_t i);
template <> __device__ __forceinline__ float ld_elem<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t *p, size_t i) { return bf16_to_f(p[i]); }

// Output formats: fp32 or bf16.
enum { kYF32 = 0, kYBF16 = 1 };

// One block of 256 threads covers NPB = min(32, 256 * PPT / C) nodes.  Threads
// 0..NPB-1 build one node's Wigner-D blocks each (fp64), shared through LDS; then
// every thread handles up to PPT (node, channel) pairs, all in registers.
template <int L> constexpr int eaas_pairs() { return L >= 3 ? 4 : 8; }
template <int L> __host__ __device__ inline int eaas_nodes_per_block(int C)
{
    return (256 * eaas_pairs<L>() / C) < 32 ? (256 * eaas_pairs<L>() / C) : 32;
}

template <int L, typename TX, int YF, bool ADJ = false>
__global__ __launch_bounds__(256) void eaas_kernel(const float *__restrict__ pos, const TX *__restrict__ x,
                                                   const float *__restrict__ path_w, int n, int C,
                                                   void *__restrict__ y_, float *__restrict__ y_deq,
                                                   float *__restrict__ dmat_out, float4 *__restrict__ pos4_out,
                                                   const Tables tabs)
{
    constexpr int NC = n_comp(L);
    constexpr int ND = n_dmat(L) > 0 ? n_dmat(L) : 1;
    constexpr int P = path_count(L);
    __shared__ float sD[32][ND];
    __shared__ int sDir[32];

    constexpr int kEaasPairs = eaas_pairs<L>();
    const int npb = eaas_nodes_per_block<L>(C);
    const int t = threadIdx.x;
    const long long node0 = (long long)blockIdx.x * npb;
    if (t < npb) {
        const long long node = node0 + t;
        if (node < n) {
            const double px = pos[3 * node + 0], py = pos[3 * node + 1], pz = pos[3 * node + 2];
            double Dd[ND];
            const bool dir = wigner_blocks<L>(px, py, pz, tabs.ds, Dd);
#pragma unroll
            for (int e = 0; e < n_dmat(L); ++e) {
                sD[t][e] = (float)Dd[e];
                if (dmat_out) dmat_out[node * n_dmat(L) + e] = (float)Dd[e];
            }
            sDir[t] = dir ? 1 : 0;
            if (pos4_out) pos4_out[node] = make_float4((float)px, (float)py, (float)pz, 1.f);
        }
    }
    __syncthreads();
    // pairs idx = t + 256 q: node ln = idx / C, channel c = idx % C
#pragma unroll
    for (int q = 0; q < kEaasPairs; ++q) {
        const int idx = t + 256 * q;
        const int ln = idx / C, c = idx - ln * C;
        const long long node = node0 + ln;
        if (ln >= npb || node >= n) continue;
        const size_t base = (size_t)node * NC * C + c;
        float xv[NC], yv[NC], w[P];
#pragma unroll
        for (int e = 0; e < NC; ++e) xv[e] = ld_elem<TX>(x, base + (size_t)e * C);
#pragma unroll
        for (int p = 0; p < P; ++p) w[p] = path_w[p * C + c];
        eaas_channel<L, ADJ>(&sD[ln][0], xv, yv, w, tabs.eaas, sDir[ln] != 0);
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            if (YF == kYBF16) {
                const uint16_t hb = f_to_bf16(yv[e]);
                reinterpret_cast<uint16_t *>(y_)[base + (size_t)e * C] = hb;
                if (y_deq) y_deq[base + (size_t)e * C] = bf16_to_f(hb);
            } else {
                reinterpret_cast<float *>(y_)[base + (size_t)e * C] = yv[e];
                if (y_deq) y_deq[base + (size_t)e * C] = yv[e];
            }
        }
    }
}

template <int L, typename TX>
static void launch_eaas_x(dim3 grid, const float *pos, const void *x, const float *path_w, int n, int C, void *y,
                          int yf, float *y_deq, float *dmat_out, float4 *pos4_out, const Tables &tb, hipStream_t stream)
{
    const TX *xp = reinterpret_cast<const TX *>(x);
    if (yf == kYBF16)
        eaas_kernel<L, TX, kYBF16><<<grid, 256, 0, stream>>>(pos, xp, path_w, n, C, y, y_deq, dmat_out, pos4_out, tb);
    else
        eaas_kernel<L, TX, kYF32><<<grid, 256, 0, stream>>>(pos, xp, path_w, n, C, y, y_deq, dmat_out, pos4_out, tb);
}

template <int L>
static hipError_t launch_eaas_l(const float *pos, const void *x, int x_bf16, const float *path_w, int n, int C,
                                void *y, int yf, float *y_deq, float *dmat_out, float4 *pos4_out, hipStream_t stream)
{
    const int npb = eaas_nodes_per_block<L>(C);
    dim3 grid((unsigned)((n + npb - 1) / npb));
    Tables tb = host_tables();
    tb.eaas = eaas_table(L);
    if (x_bf16)
        launch_eaas_x<L, uint16_t>(grid, pos, x, path_w, n, C, y, yf, y_deq, dmat_out, pos4_out, tb, stream);
    else
        launch_eaas_x<L, float>(grid, pos, x, path_w, n, C, y, yf, y_deq, dmat_out, pos4_out, tb, stream);
    return hipGetLastError();
}

hipError_t launch_eaas(int L, const float *pos, const void *x, int x_bf16, const float *path_w, int n, int C,
                       void *y, int y_format, float *y_deq, float *dmat_out, float4 *pos4_out, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    switch (L) {
    case 0: return launch_eaas_l<0>(pos, x, x_bf16, path_w, n, C, y, y_format, y_deq, dmat_out, pos4_out, stream);
    case 1: return launch_eaas_l<1>(pos, x, x_bf16, path_w, n, C, y, y_format, y_deq, dmat_out, pos4_out, stream);
    case 2: return launch_eaas_l<2>(pos, x, x_bf16, path_w, n, C, y, y_format, y_deq, dmat_out, pos4_out, stream);
    case 3: return launch_eaas_l<3>(pos, x, x_bf16, path_w, n, C, y, y_format, y_deq, dmat_out, pos4_out, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int L>
static hipError_t launch_eaas_adj_l(const float *pos, const float *x, const float *path_w, int n, int C, float *y,
                                    hipStream_t stream)
{
    const int npb = eaas_nodes_per_block<L>(C);
    dim3 grid((unsigned)((n + npb - 1) / npb));
    Tables tb = host_tables();
    tb.eaas = eaas_table(L);
    eaas_kernel<L, float, kYF32, true><<<grid, 256, 0, stream>>>(pos, x, path_w, n, C, y, nullptr, nullptr, nullptr, tb);
    return hipGetLastError();
}

hipError_t launch_eaas_adjoint(int L, const float *pos, const float *x, const float *path_w, int n, int C, float *y,
                               hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    switch (L) {
    case 0: return launch_eaas_adj_l<0>(pos, x, path_w, n, C, y, stream);
    case 1: return launch_eaas_adj_l<1>(pos, x, path_w, n, C, y, stream);
    case 2: return launch_eaas_adj_l<2>(pos, x, path_w, n, C, y, stream);
    case 3: return launch_eaas_adj_l<3>(pos, x, path_w, n, C, y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
