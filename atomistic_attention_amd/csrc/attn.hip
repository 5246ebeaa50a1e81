// Streaming neighbour attention for 16-bit storage (the general kernel: any l_max,
// any size; attn_pair.hip serves l_max <= 2 below its size limit, attn_f32.hip
// serves fp32 storage).  It stops at the normalised message m_i.
//
// E2Former-V2 explainer, section 3.1 (node-centric message passing: the
// message m_i = sum_j alpha_ij h'_j is formed on the fly, then coupled with the
// target's own encoding) and section 3.2 (Algorithm 1: online softmax with a
// running maximum and normaliser, each key/value row read once, accumulation
// on chip, one target per independent work item, padded neighbours skipped).
// The distance bias -- distance, Gaussian expansion and cosine envelope
// computed in the kernel and never written out -- follows the FlashSchNet
// page, section 2.1; target-owned rows with no atomics follow its section 2.3.
//
// Mapping (one 64-lane wave per target atom i; H heads of 8 channels):
//   * lane = u * 2H + b * H + h: head h, channel half b (channels 8h + 4b .. +4 of
//     every (l, m) component, so a lane keeps n_comp * 4 fp32 accumulators) and
//     neighbour slot u of PS = 32 / H slots streamed side by side;
//   * neighbours are taken 16 at a time; slot u streams S = H / 2 consecutive
//     pairs of the chunk with its own running max / normaliser / accumulators;
//   * the distance bias of the 16 pairs for every head is one small product
//     phi[16 pairs x R] . W_rbf[R x 16 heads] on the matrix cores
//     (v_mfma_f32_16x16x4_f32, fp32): lane l evaluates phi_k(d_p) for pair
//     p = l % 16 and k = l / 16 + 4 kk, i.e. every Gaussian exactly once, and the
//     product lands in the lanes (or, for 16 heads, the lane pair) that need it;
//   * q . k is a 4-channel partial per lane plus one swap with the other half;
//   * per chunk: indices come from registers prefetched one chunk ahead, every
//     key row and half the value rows are requested at once, the bias math runs
//     while they are in flight, the second half of the value rows is requested
//     as soon as the first half is consumed;
//   * at the end the PS partial softmaxes are merged by a butterfly that halves
//     the channel set at each step (reduce-scatter), leaving every lane whole
//     channels, and the lane writes its channels of the normalised message m_i,
//     which the output-projection kernel couples.
// Value rows are read as 16-byte pieces (4 channels of two interleaved fp16
// components, plus an 8-byte piece of an odd last component); the 2H lanes of a
// slot cover a contiguous stretch of the neighbour's row.  The key arrives in fp32
// (16 bytes per lane), so the logits carry no 16-bit rounding, and a neighbour's
// h' carries one power-of-two scale (pos4[j].w): it is folded into the softmax
// weight of the pair, so each value element costs one mixed-precision FMA.
#include "attn_common.h"

namespace e2v2 {

template <int L, int H>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_kernel(const AttnArgs A)
{
    constexpr int NC = n_comp(L);
    constexpr int C = 8 * H;
    constexpr int PS = 32 / H;          // neighbour slots per wave
    constexpr int S = H / 2;            // pairs per slot per 16-pair chunk
    constexpr int NB = Log2<PS>::v;
    constexpr float LOG2E = 1.4426950408889634f;
    // Value rows are fetched in NPH phases of SP steps, each phase sized to about
    // 72 registers (one 8- or 16-byte piece per component and step) when a step's
    // piece is small, else to one step.
    constexpr int RPR = 2;
    constexpr int BUDGET = NC * RPR <= 18 ? 72 : 40;
    constexpr int SPF = BUDGET / (NC * RPR) > 0 ? BUDGET / (NC * RPR) : 1;
    constexpr int SP = SPF >= 8 && S >= 8 ? 8 : SPF >= 4 && S >= 4 ? 4 : SPF >= 2 && S >= 2 ? 2 : 1;
    constexpr int NPH = S / SP;

    const int lane = threadIdx.x & 63;
    // Workgroups are handed to the 8 XCDs round robin; give each XCD one contiguous
    // run of target slots so that, with a spatial target order, the targets one
    // XCD works on at a time are close together and share rows in its L2.
    const int nb = gridDim.x, xcd = blockIdx.x & 7, kth = blockIdx.x >> 3;
    const int lb = xcd * (nb >> 3) + (xcd < (nb & 7) ? xcd : (nb & 7)) + kth;
    const int slot = __builtin_amdgcn_readfirstlane(lb * 4 + (int)(threadIdx.x >> 6));
    const int n = A.n;
    int i = slot;
    if (A.order && slot < n) i = __builtin_amdgcn_readfirstlane(A.order[slot]);
    const int h = lane % H, b = (lane / H) & 1, u = lane / (2 * H);
    const int kq = lane >> 4, pm = lane & 15;
    const int R = A.R;
    const int KK = (R + 3) >> 2;
    const int cb = 8 * h + 4 * b;       // first channel of this lane

    // B operand of the bias product, log2(e) W_rbf[k][head] zero-padded to 64 x 16,
    // in LDS: the product is the bias in the log2 domain of the softmax.
    __shared__ float sW[64 * 16];
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
        const int k = e >> 4, hh = (e & 15) % H;
        sW[e] = (k < R) ? A.w_rbf[k * H + hh] * LOG2E : 0.f;
    }
    __syncthreads();
    if (slot >= n || i < 0 || i >= n) return;             // whole wave: i is wave-uniform

    const float4 pi4 = A.pos4[i];
    const float4 qv = *reinterpret_cast<const float4 *>(A.q + (size_t)i * C + cb);
    const float qscale = LOG2E * 0.35355339059327373f;   // log2(e) / sqrt(8)
    const int start = __builtin_amdgcn_readfirstlane(A.nbr_start[i]);
    const int len = __builtin_amdgcn_readfirstlane(A.nbr_len[i]);
    // Gaussians in the log2 domain: exp(-t^2 / 2) = exp2(-(g t)^2) with g^2 = log2(e) / 2,
    // t = (d - mu_k) / Delta; the envelope joins the exponent as log2(fc).
    const float gsc = 0.84932180028801904f;              // sqrt(log2(e) / 2)
    const float inv_delta = gsc * (float)(R - 1) / A.cutoff;
    const float cos_scale = 0.5f / A.cutoff;             // cos(pi d / rc) = cos(2 pi * d / (2 rc))

    float mu = -1e30f, z = 0.f;
    float acc[NC][4];
#pragma unroll
    for (int e = 0; e < NC; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[e][c] = 0.f;

    // Prologue: pair pm of the first chunk (index and padded position).
    int jp = -1;
    float4 pj = make_float4(0.f, 0.f, 0.f, 0.f);
    if (pm < len) jp = A.nbr_idx[start + pm];
    if (jp >= 0 && jp < n) pj = A.pos4[jp];

    for (int c0 = 0; c0 < len; c0 += 16) {
        // ---- (a) this lane's S neighbours of the chunk and their row scales
        int js[S];
        float scl[S];                  // the neighbours' h' scale (16-bit storage)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int p = u * S + s;
            const int j = __shfl(jp, p, 64);
            js[s] = (j >= 0 && j < n) ? j : -1;
            scl[s] = __shfl(pj.w, p, 64);
        }
        // ---- (b) issue every key row (fp32) and the first phase of value rows
        float4 kv[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const size_t node = (size_t)(js[s] >= 0 ? js[s] : i);
            kv[s] = *reinterpret_cast<const float4 *>(A.k + node * C + cb);
        }
        HpStep<true, NC> hv[SP];
#pragma unroll
        for (int s = 0; s < SP; ++s) hv[s].load(A.hp, js[s] >= 0 ? js[s] : i, cb, C);
        // ---- (c) prefetch the next chunk's index for pair pm
        int jn = -1;
        if (c0 + 16 + pm < len) jn = A.nbr_idx[start + c0 + 16 + pm];
        // ---- (d) pair pm: distance, Gaussians x envelope, bias product on the matrix cores
        const bool vp = (jp >= 0) && (jp < n);
        const float dx = pj.x - pi4.x, dy = pj.y - pi4.y, dz = pj.z - pi4.z;
        const float d = vp ? __builtin_amdgcn_sqrtf(dx * dx + dy * dy + dz * dz) : 0.f;   // v_sqrt_f32, 1 ulp
        const float fc = (vp && d < A.cutoff) ? 0.5f * (__builtin_amdgcn_cosf(d * cos_scale) + 1.f) : 0.f;   // cutoff mask
        const float lfc = __builtin_amdgcn_logf(fmaxf(fc, 0.f));   // log2; fc = 0 gives -inf, phi = 0
        const float t0 = fmaf(d, inv_delta, -gsc * (float)kq);   // g (d - mu_k) / Delta for k = kq
        const float *wrow = sW + kq * 16 + pm;
        floatx4 bias = {0.f, 0.f, 0.f, 0.f};
        // Branch-free product over 8 (up to 32 RBFs) or 16 steps of 4 RBFs; the
        // padded LDS rows are zero, so surplus Gaussians contribute nothing.
        if (KK <= 8) {
            float wk[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) wk[kk] = wrow[64 * kk];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const float tk = t0 - (4.0f * gsc) * (float)kk;
                const float phi = __builtin_amdgcn_exp2f(fmaf(-tk, tk, lfc));
                bias = __builtin_amdgcn_mfma_f32_16x16x4f32(phi, wk[kk], bias, 0, 0, 0);
            }
        } else {
            float wk[16];
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) wk[kk] = wrow[64 * kk];
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const float tk = t0 - (4.0f * gsc) * (float)kk;
                const float phi = __builtin_amdgcn_exp2f(fmaf(-tk, tk, lfc));
                bias = __builtin_amdgcn_mfma_f32_16x16x4f32(phi, wk[kk], bias, 0, 0, 0);
            }
        }
        // bias[r] holds pair 4 (lane / 16) + r for head (lane % 16) % H.
        float bs[S];
        if constexpr (H == 16) {            // pairs 8u .. 8u+7: half b holds 4b .. 4b+3, the partner the rest
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float other = __shfl_xor(bias[r], 16, 64);
                bs[r] = b ? other : bias[r];
                bs[4 + r] = b ? bias[r] : other;
            }
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s) bs[s] = pick4(bias, ((u * S) & 3) + s);
        }
        // ---- (e) logits (4-channel partial + the other half) and the online-softmax update
        float sl[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            float qk = qv.x * kv[s].x;
            qk = fmaf(qv.y, kv[s].y, qk);
            qk = fmaf(qv.z, kv[s].z, qk);
            qk = fmaf(qv.w, kv[s].w, qk);
            qk += __shfl_xor(qk, H, 64);
            sl[s] = js[s] >= 0 ? fmaf(qk, qscale, bs[s]) : -INFINITY;
        }
        // The reference maximum mu moves only when a logit exceeds it by more than 8
        // (weights up to 2^8 are harmless in fp32), so the rescale of the
        // accumulators is skipped in most chunks; the branch is wave-uniform.
        float mx = sl[0];
#pragma unroll
        for (int s = 1; s < S; ++s) mx = fmaxf(mx, sl[s]);
        const bool grow = mx > mu + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float mun = grow ? mx : mu;
            const float corr = __builtin_amdgcn_exp2f(mu - mun);
            z *= corr;
#pragma unroll
            for (int e = 0; e < NC; ++e)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[e][c] *= corr;
            mu = mun;
        }
        float ps[S];
        float psum = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            ps[s] = __builtin_amdgcn_exp2f(sl[s] - mu);
            psum += ps[s];
            ps[s] *= scl[s];                   // fold the row scale into the weight
        }
        z += psum;
        // ---- (f) accumulate phase by phase; the next chunk's position is requested
        //          with the last phase
        float4 pjn = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            if (ph > 0) {
                __builtin_amdgcn_sched_barrier(0);     // this phase reuses the previous phase's registers
#pragma unroll
                for (int s = 0; s < SP; ++s) hv[s].load(A.hp, js[ph * SP + s] >= 0 ? js[ph * SP + s] : i, cb, C);
            }
            if (ph == NPH - 1 && jn >= 0 && jn < n) pjn = A.pos4[jn];
#pragma unroll
            for (int e = 0; e < NC; ++e)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float a = acc[e][c];
#pragma unroll
                    for (int s = 0; s < SP; ++s) a = fmaf(ps[ph * SP + s], hv[s].get(e, c), a);
                    acc[e][c] = a;
                }
        }
        pj = pjn;
        jp = jn;
    }

    // ---- merge the PS partial softmaxes (butterfly over the slot bits of the lane)
    int off = 0;
#pragma unroll
    for (int st = 0; st < NB; ++st) {
        const int bit = NB - 1 - st;
        const int mask = (2 * H) << bit;
        const float mo = __shfl_xor(mu, mask, 64);
        const float mun = fmaxf(mu, mo);
        const float corr = __builtin_amdgcn_exp2f(mu - mun);
        mu = mun;
        z *= corr;
        z += __shfl_xor(z, mask, 64);
        const bool upper = ((u >> bit) & 1) != 0;
        if (st < 2) {                       // 4 -> 2 -> 1 channels
            const int half = 2 >> st;
#pragma unroll
            for (int e = 0; e < NC; ++e)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    if (c < half) {
                        const float lo = acc[e][c] * corr, hi = acc[e][c + half] * corr;
                        const float keep = upper ? hi : lo;
                        const float send = upper ? lo : hi;
                        acc[e][c] = keep + __shfl_xor(send, mask, 64);
                    }
                }
            off += upper ? half : 0;
        } else {                            // one channel left: plain sum
#pragma unroll
            for (int e = 0; e < NC; ++e) {
                const float v = acc[e][0] * corr;
                acc[e][0] = v + __shfl_xor(v, mask, 64);
            }
        }
    }
    constexpr int NCH = (NB >= 2) ? 1 : (4 >> NB);
    const bool writer = (NB <= 2) || ((u & 1) == 0);

    // store the normalised message m_i (fp16 under a node scale); the target
    // coupling runs in the output-projection kernel, on whole nodes
    store_message_f16<NC, NCH>(A, i, C, z, acc, cb + off, writer, lane);
}

template <int L>
static hipError_t launch_attn_lh(const AttnArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.n + 3) / 4)), block(256);
    switch (a.H) {
    case 4: attn_kernel<L, 4><<<grid, block, 0, stream>>>(a); break;
    case 8: attn_kernel<L, 8><<<grid, block, 0, stream>>>(a); break;
    case 16: attn_kernel<L, 16><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn(int L, int hp_bf16, const AttnArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    if (!hp_bf16) return launch_attn_f32(L, a, stream);     // fp32 storage: attn_f32.hip
    if (hp_quad_layout(L, a.H, a.C, a.n)) return launch_attn_quad(L, a, stream);
    if (L <= 2 && a.n < attn_pair_max_atoms(L, 8 * a.H)) return launch_attn_pair(L, a, stream);
    switch (L) {
    case 0: return launch_attn_lh<0>(a, stream);
    case 1: return launch_attn_lh<1>(a, stream);
    case 2: return launch_attn_lh<2>(a, stream);
    case 3: return launch_attn_lh<3>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
