// Streaming neighbour attention, two targets per wave (16-bit storage, l_max <= 2).
//
// E2Former-V2 explainer, section 3.1 (the message m_i = sum_j alpha_ij h'_j is
// formed on the fly) and section 3.2 (Algorithm 1: online softmax with a running
// maximum and normaliser, each key/value row read once, accumulation on chip,
// padded neighbours skipped).  The distance bias -- distance, Gaussian expansion
// and cosine envelope computed in the kernel, never written out -- follows the
// FlashSchNet page, section 2.1; target-owned rows with no atomics follow its
// section 2.3.
//
// Neighbouring targets share most of their neighbours.  A wave takes the two
// targets at processing slots 2 w and 2 w + 1 (spatially close when the order
// comes from the cell list) and streams the union of their two lists: every
// neighbour row is loaded once and feeds both targets, each with its own logit,
// bias, online softmax and accumulators.  At 32,768 atoms and an 8 A cutoff the
// union of two consecutive targets' lists is 1.27 times one list, so a pair of
// (target, neighbour) costs 0.64 of the row loads of one target per wave.
//
// The union is built in LDS before the stream: the wave sorts the two lists'
// entries (atom, list) in registers (one bitonic merge when both lists ascend, the
// full sort otherwise); an entry of the first list directly followed
// by the same atom from the second list becomes one entry for both targets, and
// invalid indices (negative or >= n) drop out.  An atom listed twice in one list
// stays two entries, so it counts twice, as in the per-target kernel.  Entries
// are laid out as three segments (both lists, first only, second only), so a
// 16-entry chunk nearly always feeds one fixed set of targets and the work of a
// target with no entry in the chunk (bias, logits, softmax, accumulation) is
// skipped wave-wide: the arithmetic per (target, neighbour) pair stays that of
// the per-target kernel while the row loads drop.  When the two lists hold more
// than kPairUnionMax entries together, the wave streams the first list and then
// the second instead (correct, without the sharing).
//
// Lane mapping, chunking, the bias product on the matrix cores, the value-row
// layout and the final reduce-scatter are those of attn_kernel (attn.hip):
// lane = u * 2H + b * H + h owns 4 channels of head h in neighbour slot u and now
// keeps two sets of accumulators, one per target.
#include "attn_common.h"

#include <climits>

namespace e2v2 {

namespace {

constexpr int kPairUnionMax = 512;            // list entries a wave merges in LDS

// Stream entry code: (j << 2) | (in the first list) << 1 | (in the second list);
// -1 for an entry that contributes to neither target.  Requires n < 2^29.
__device__ __forceinline__ int entry_code(int j, bool fa, bool fb)
{
    return (j << 2) | (fa ? 2 : 0) | (fb ? 1 : 0);
}

// The union of the two lists, written to su[0 .. return value).  Keys are
// (j << 1) | list; invalid entries sort last and are dropped.  The first list
// fills positions [0, la) and the second, reversed, [64 E - lb, 64 E): when both
// lists ascend the keys already form a bitonic sequence and the last merge phase
// of the network sorts them; any other lists (the neighbour builder writes its
// rows in its scan order) take the full sort.
template <int E>
__device__ __forceinline__ int pair_union(const int32_t *__restrict__ idx, int n, int sa, int la, int sb, int lb,
                                          int *su, int lane)
{
    constexpr int N = 64 * E;
    int key[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int x = lane * E + k;
        int kv = INT_MAX;
        if (x < la) {
            const int j = idx[sa + x];
            if (j >= 0 && j < n) kv = j << 1;
        } else if (x >= N - lb) {
            const int j = idx[sb + (N - 1 - x)];
            if (j >= 0 && j < n) kv = (j << 1) | 1;
        }
        key[k] = kv;
    }
    {
        const int nxt0 = __shfl_down(key[0], 1, 64);
        bool bad = false;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int x = lane * E + k;
            const int nx = k < E - 1 ? key[k + 1] : nxt0;
            bad |= (x + 1 < la && key[k] > nx) || (x >= N - lb && x + 1 < N && key[k] < nx);
        }
        if (__builtin_amdgcn_ballot_w64(bad) == 0) wave_bitonic_merge<E>(key, lane);
        else wave_bitonic_sort<E>(key, lane);
    }
    const int prev_last = __shfl_up(key[E - 1], 1, 64);
    const int next_first = __shfl_down(key[0], 1, 64);
    int code[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int kv = key[k];
        const int prv = k > 0 ? key[k - 1] : (lane > 0 ? prev_last : INT_MAX);
        const int nxt = k < E - 1 ? key[k + 1] : (lane < 63 ? next_first : INT_MAX);
        int c = -1;
        if (kv != INT_MAX) {
            if ((kv & 1) == 0) c = entry_code(kv >> 1, true, nxt == (kv | 1));   // first list (+ second)
            else if (prv != (kv & ~1)) c = entry_code(kv >> 1, false, true);     // second list only
        }
        code[k] = c;
    }
    // Three segments -- atoms of both lists, of the first only, of the second only,
    // each in increasing atom order -- so that most 16-entry chunks feed one
    // target or both throughout and the kernel skips a target's work wave-wide.
    int cnt[3] = {0, 0, 0};
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int m = code[k] & 3;
        if (code[k] >= 0) cnt[m == 3 ? 0 : m == 2 ? 1 : 2] += 1;
    }
    int pos[3], tot3[3];
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        int incl = cnt[g];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        pos[g] = incl - cnt[g];
        tot3[g] = __shfl(incl, 63, 64);
    }
    pos[1] += tot3[0];
    pos[2] += tot3[0] + tot3[1];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (code[k] < 0) continue;
        const int m = code[k] & 3;
        const int g = m == 3 ? 0 : m == 2 ? 1 : 2;
        su[pos[g]++] = code[k];
    }
    return tot3[0] + tot3[1] + tot3[2];
}

// v_permlane16_swap_b32 on a and b.  In each pair of 16-lane rows (2 t, 2 t + 1), lane
// for lane, the even row ends with (a, b) = (its own a, the odd row's a) and the odd row
// with (the even row's b, its own b).
__device__ __forceinline__ void row_swap(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void pair_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

// Entry codes need n < 2^29, and rows are addressed by 32-bit byte offsets: n times
// the longest row (h' 2 NC C bytes, k 4 C, position 16) stays below 2^32.
long long attn_pair_max_atoms(int L, int C)
{
    const long long nc = (long long)(L + 1) * (L + 1);
    long long row = 2 * nc * C;
    if (row < 4LL * C) row = 4LL * C;
    if (row < 16) row = 16;
    const long long lim = (1LL << 32) / row;
    return lim < (1LL << 29) ? lim : (1LL << 29);
}

template <int L, int H>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_pair_kernel(const AttnArgs A)
{
    constexpr int NC = n_comp(L);
    constexpr int C = 8 * H;
    constexpr int PS = 32 / H;          // neighbour slots per wave
    constexpr int S = H / 2;            // entries per slot per 16-entry chunk
    constexpr int NB = Log2<PS>::v;
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int SP = S >= 2 ? 2 : 1;  // value rows per phase
    constexpr int NPH = S / SP;
    // With H = 16 the two channel halves b of a head sit in adjacent 16-lane rows, and
    // each half computes the logits and softmax weights of 4 of its slot's 8 entries.
    constexpr bool ROWHALF = H == 16;
    constexpr int SO = ROWHALF ? 4 : S;  // entries whose logit this lane computes

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // Workgroups go to the 8 XCDs round robin; each XCD gets one contiguous run of
    // target pairs, so the targets one XCD works on at a time are close together
    // and share rows in its L2.
    const int nb = gridDim.x, xcd = blockIdx.x & 7, kth = blockIdx.x >> 3;
    const int lb = xcd * (nb >> 3) + (xcd < (nb & 7) ? xcd : (nb & 7)) + kth;
    const int ps = __builtin_amdgcn_readfirstlane(lb * 4 + wv);
    const int n = A.n;
    const int h = lane % H, b = (lane / H) & 1, u = lane / (2 * H);
    const int kq = lane >> 4, pm = lane & 15;
    const int R = A.R;
    const int cb = 8 * h + 4 * b;       // first channel of this lane

    // B operand of the bias product in fp16, log2(e) W_rbf[k][head] zero-padded to
    // 64 x 16, as v_mfma_f32_16x16x32_f16 fragments: group g, lane l holds
    // k = 32 g + 8 (l / 16) + i (i < 8) for head column l % 16.
    __shared__ __align__(16) _Float16 sWh[2][64][8];
    __shared__ int sU[4][kPairUnionMax];
    __shared__ __align__(16) int sE[4][16];      // the chunk's entries, per wave
    __shared__ __align__(16) float sS[4][16];    // and their row scales
    for (int e = threadIdx.x; e < 2 * 64 * 8; e += 256) {
        const int g = e >> 9, l = (e >> 3) & 63, i = e & 7;
        const int k = 32 * g + 8 * (l >> 4) + i, hh = (l & 15) % H;
        sWh[g][l][i] = (_Float16)((k < R) ? A.w_rbf[k * H + hh] * LOG2E : 0.f);
    }
    __syncthreads();

    // ---- the two targets and their lists (everything here is wave-uniform)
    const int s0 = 2 * ps;
    if (s0 >= n) return;
    int ia = s0, ib = s0 + 1 < n ? s0 + 1 : -1;
    if (A.order) {
        ia = A.order[s0];
        if (ib >= 0) ib = A.order[s0 + 1];
    }
    ia = __builtin_amdgcn_readfirstlane(ia);
    ib = __builtin_amdgcn_readfirstlane(ib);
    const bool va = ia >= 0 && ia < n, vb = ib >= 0 && ib < n;
    if (!va && !vb) return;
    const int sa = va ? __builtin_amdgcn_readfirstlane(A.nbr_start[ia]) : 0;
    const int la0 = va ? __builtin_amdgcn_readfirstlane(A.nbr_len[ia]) : 0;
    const int sb = vb ? __builtin_amdgcn_readfirstlane(A.nbr_start[ib]) : 0;
    const int lb0 = vb ? __builtin_amdgcn_readfirstlane(A.nbr_len[ib]) : 0;
    const int la = la0 > 0 ? la0 : 0, lbn = lb0 > 0 ? lb0 : 0;
    const long long tot64 = (long long)la + lbn;
    const int tot = tot64 < INT_MAX ? (int)tot64 : INT_MAX;
    const int ifill = va ? ia : ib;     // row read for entries that feed no target

    int *su = sU[wv];
    const bool uni = tot <= kPairUnionMax;
    int nu = tot;
    if (uni) {
        if (tot <= 64) nu = pair_union<1>(A.nbr_idx, n, sa, la, sb, lbn, su, lane);
        else if (tot <= 128) nu = pair_union<2>(A.nbr_idx, n, sa, la, sb, lbn, su, lane);
        else if (tot <= 256) nu = pair_union<4>(A.nbr_idx, n, sa, la, sb, lbn, su, lane);
        else nu = pair_union<8>(A.nbr_idx, n, sa, la, sb, lbn, su, lane);
        nu = __builtin_amdgcn_readfirstlane(nu);
        pair_lds_sync();
    }
    // entry x < nu of the stream
    auto entry = [&](int x) -> int {
        if (uni) return su[x];
        const bool fa = x < la;
        const int j = A.nbr_idx[fa ? sa + x : sb + (x - la)];
        return (j >= 0 && j < n) ? entry_code(j, fa, !fa) : -1;
    };

    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    // loads from valid rows only, then the value is masked
    const int ra = va ? ia : ifill, rb = vb ? ib : ifill;
    const float4 pa0 = A.pos4[ra], pb0 = A.pos4[rb];
    const float4 qa0 = *reinterpret_cast<const float4 *>(A.q + (size_t)ra * C + cb);
    const float4 qb0 = *reinterpret_cast<const float4 *>(A.q + (size_t)rb * C + cb);
    const float4 pa = va ? pa0 : zero4, pb = vb ? pb0 : zero4;
    const float4 qa = va ? qa0 : zero4, qb = vb ? qb0 : zero4;
    const float qscale = LOG2E * 0.35355339059327373f;   // log2(e) / sqrt(8)
    // Gaussians in the log2 domain: exp(-t^2 / 2) = exp2(-(g t)^2) with g^2 = log2(e) / 2,
    // t = (d - mu_k) / Delta; the envelope joins the exponent as log2(fc).
    const float gsc = 0.84932180028801904f;              // sqrt(log2(e) / 2)
    const float inv_delta = gsc * (float)(R - 1) / A.cutoff;
    const float cos_scale = 0.5f / A.cutoff;             // cos(pi d / rc) = cos(2 pi * d / (2 rc))

    float mua = -1e30f, za = 0.f, mub = -1e30f, zb = 0.f;
    float acca[NC][4], accb[NC][4];
#pragma unroll
    for (int e = 0; e < NC; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acca[e][c] = 0.f;
            accb[e][c] = 0.f;
        }

    // Bias of pair pm of the chunk (position pj) for the target at pt, in lanes
    // (4 (lane / 16) + r, head (lane % 16) % H) of the returned product.
    auto bias_of = [&](float4 pj, float4 pt, bool ok) -> floatx4 {
        const float dx = pj.x - pt.x, dy = pj.y - pt.y, dz = pj.z - pt.z;
        const float d = ok ? __builtin_amdgcn_sqrtf(dx * dx + dy * dy + dz * dz) : 0.f;   // v_sqrt_f32, 1 ulp
        const float fc = (ok && d < A.cutoff) ? 0.5f * (__builtin_amdgcn_cosf(d * cos_scale) + 1.f) : 0.f;   // cutoff mask
        const float lfc = __builtin_amdgcn_logf(fmaxf(fc, 0.f));   // log2; fc = 0 gives -inf, phi = 0
        // g (d - mu_k) / Delta for k = 8 kq; past the cutoff phi is 0 whatever t is, and
        // the clamp keeps the ratio below finite for listed pairs far beyond it
        const float t0 = fmaf(fminf(d, A.cutoff), inv_delta, -gsc * (float)(8 * kq));
        // A operand: lane (kq, pm) holds phi_k of pair pm for k = 8 kq + i (+ 32)
        // With t_i = t - g i (g = gsc), phi_{i+1} / phi_i = exp2(2 g t - g^2) e^{-i}: two
        // exponentials and a product chain give the lane's 8 consecutive Gaussians.
        // Whenever one of them exceeds 2^-24 the first is above 2^-118, a normal
        // number, so the chain loses nothing that matters.
        auto group = [&](int g, floatx4 acc) {
            const float t = t0 - gsc * (float)(32 * g);
            float phi = __builtin_amdgcn_exp2f(fmaf(-t, t, lfc));
            float r = __builtin_amdgcn_exp2f(fmaf(2.f * gsc, t, -gsc * gsc));
            half8_t a;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a[i] = (_Float16)phi;
                phi *= r;
                r *= 0.36787944117144233f;                      // exp2(-2 g^2) = 1 / e
            }
            const half8_t w = *reinterpret_cast<const half8_t *>(&sWh[g][lane][0]);
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, w, acc, 0, 0, 0);
        };
        floatx4 bias = group(0, floatx4{0.f, 0.f, 0.f, 0.f});
        if (R > 32) bias = group(1, bias);
        return bias;
    };
    // this lane's S pair biases from the product (H < 16: pairs u S .. u S + S - 1 lie
    // in this lane's four)
    auto lane_bias = [&](const floatx4 &bias, float (&bs)[S]) {
#pragma unroll
        for (int s = 0; s < S; ++s) bs[s] = pick4(bias, ((u * S) & 3) + s);
    };
    // lazily moved reference maximum (as in attn_kernel), then the chunk's weights
    auto softmax = [&](const float (&sl)[SO], const float (&scl)[SO], float &mu, float &z, float (&acc)[NC][4],
                       float (&p)[S]) {
        float mx = sl[0];
#pragma unroll
        for (int s = 1; s < SO; ++s) mx = fmaxf(mx, sl[s]);
        if constexpr (ROWHALF) {                // one maximum for both halves of the slot
            float me = mx, mo = mx;
            row_swap(me, mo);
            mx = fmaxf(me, mo);
        }
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
        float psum = 0.f, po[SO];
#pragma unroll
        for (int s = 0; s < SO; ++s) {
            po[s] = __builtin_amdgcn_exp2f(sl[s] - mu);
            psum += po[s];
            po[s] *= scl[s];                   // fold the row scale into the weight
        }
        z += psum;                             // with row halves: this half's entries only
        if constexpr (ROWHALF) {               // every lane takes all 8 weights of its slot
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pe = po[r], pw = po[r];
                row_swap(pe, pw);
                p[r] = pe;
                p[4 + r] = pw;
            }
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s) p[s] = po[s];
        }
    };

    // Prologue: entry and position of pair pm of the first chunk.
    int ep = -1;
    float4 pj = zero4;
    if (pm < nu) ep = entry(pm);
    if (ep >= 0) pj = A.pos4[ep >> 2];

    for (int c0 = 0; c0 < nu; c0 += 16) {
        // ---- (a) the chunk's entries and row scales pass from the pair lanes through
        //          LDS; every lane reads the S entries of its slot
        if (lane < 16) {
            sE[wv][lane] = ep;
            sS[wv][lane] = pj.w;
        }
        pair_lds_sync();
        uint32_t rw[S];                         // rows to load (an entry of neither target reads ifill's)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int e = sE[wv][u * S + s];
            rw[s] = uint32_t(e >= 0 ? (e >> 2) : ifill);
        }
        // Entries whose logit and softmax weight this lane computes: all S of the slot,
        // or with row halves the 4 entries 4 b + r of its half.
        const int s0o = ROWHALF ? 4 * b : 0;
        bool fa[SO], fb[SO];
        float scl[SO];
#pragma unroll
        for (int r = 0; r < SO; ++r) {
            const int e = sE[wv][u * S + s0o + r];
            fa[r] = e >= 0 && (e & 2) != 0;
            fb[r] = e >= 0 && (e & 1) != 0;
            scl[r] = sS[wv][u * S + s0o + r];
        }
        // ---- (b) every key row (fp32) and the first phase of value rows
        float4 kf[S];
#pragma unroll
        for (int s = 0; s < S; ++s)
            kf[s] = *reinterpret_cast<const float4 *>(reinterpret_cast<const unsigned char *>(A.k) +
                                                      (rw[s] * uint32_t(4 * C) + uint32_t(4 * cb)));
        HpStep<true, NC> hv[2][SP];       // value rows, double-buffered across phases
#pragma unroll
        for (int s = 0; s < SP; ++s) hv[0][s].load32(A.hp, rw[s], cb, C);
        // ---- (c) the next chunk's entry for pair pm
        int en = -1;
        if (c0 + 16 + pm < nu) en = entry(c0 + 16 + pm);
        // ---- (d) which targets this chunk feeds (wave-uniform), and the bias of
        //          pair pm for them
        const bool vp = ep >= 0;
        const bool anya = __builtin_amdgcn_ballot_w64(vp && (ep & 2) != 0) != 0;
        const bool anyb = __builtin_amdgcn_ballot_w64(vp && (ep & 1) != 0) != 0;
        // ---- (e) per target: logits (4-channel partial + the other half) and the
        //          online-softmax update
        auto logits = [&](float4 pt, bool ok, float4 qv, const bool (&f)[SO], float (&sl)[SO]) {
            const floatx4 bias = bias_of(pj, pt, vp && ok);
            float x[S];                         // this half's 4-channel part of q . k
#pragma unroll
            for (int s = 0; s < S; ++s) {
                float qk = qv.x * kf[s].x;
                qk = fmaf(qv.y, kf[s].y, qk);
                qk = fmaf(qv.z, kf[s].z, qk);
                x[s] = fmaf(qv.w, kf[s].w, qk);
            }
            if constexpr (ROWHALF) {
                // Half 0 takes entry r's full dot product and half 1 entry 4 + r's;
                // the bias product already holds pairs 8 u + 4 b + r in this lane.
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float lo = x[r], hi = x[4 + r];
                    row_swap(lo, hi);
                    sl[r] = f[r] ? fmaf(lo + hi, qscale, bias[r]) : -INFINITY;
                }
            } else {
                float bs[S];
                lane_bias(bias, bs);
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float qk = x[s] + __shfl_xor(x[s], H, 64);
                    sl[s] = f[s] ? fmaf(qk, qscale, bs[s]) : -INFINITY;
                }
            }
        };
        float psa[S], psb[S];
        if (anya) {
            float sl[SO];
            logits(pa, va, qa, fa, sl);
            softmax(sl, scl, mua, za, acca, psa);
        }
        if (anyb) {
            float sl[SO];
            logits(pb, vb, qb, fb, sl);
            softmax(sl, scl, mub, zb, accb, psb);
        }
        // ---- (f) accumulate phase by phase, the rows of phase ph + 1 in flight while
        //          phase ph is summed; the next chunk's position is requested with the
        //          last phase
        float4 pjn = zero4;
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            if (ph > 0) {
                // phase ph - 1 is summed before its buffer takes the rows of phase ph + 1
#pragma unroll
                for (int e = 0; e < NC; ++e) {
                    asm volatile("" : "+v"(acca[e][0]), "+v"(acca[e][1]), "+v"(acca[e][2]), "+v"(acca[e][3])::"memory");
                    asm volatile("" : "+v"(accb[e][0]), "+v"(accb[e][1]), "+v"(accb[e][2]), "+v"(accb[e][3])::"memory");
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (ph + 1 < NPH) {
#pragma unroll
                for (int s = 0; s < SP; ++s) hv[(ph + 1) & 1][s].load32(A.hp, rw[(ph + 1) * SP + s], cb, C);
            }
            if (ph == NPH - 1 && en >= 0)
                pjn = *reinterpret_cast<const float4 *>(reinterpret_cast<const unsigned char *>(A.pos4) +
                                                        uint32_t(en >> 2) * 16u);
            auto accumulate = [&](const float (&p)[S], float (&acc)[NC][4]) {
#pragma unroll
                for (int e = 0; e < NC; ++e)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float a = acc[e][c];
#pragma unroll
                        for (int s = 0; s < SP; ++s) a = fmaf(p[ph * SP + s], hv[ph & 1][s].get(e, c), a);
                        acc[e][c] = a;
                    }
            };
            if (anya) accumulate(psa, acca);
            if (anyb) accumulate(psb, accb);
        }
        pj = pjn;
        ep = en;
    }

    // ---- merge the PS partial softmaxes of each target (butterfly over the slot
    //      bits of the lane, halving the channel set at each step) and store m
    auto merge = [&](float &mu, float &z, float (&acc)[NC][4]) {
        if constexpr (ROWHALF) {                // the two halves' normalisers (same maximum)
            float ze = z, zo = z;
            row_swap(ze, zo);
            z = ze + zo;
        }
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
            } else {                            // one channel left: plain sum
#pragma unroll
                for (int e = 0; e < NC; ++e) {
                    const float v = acc[e][0] * corr;
                    acc[e][0] = v + __shfl_xor(v, mask, 64);
                }
            }
        }
    };
    int off = 0;
#pragma unroll
    for (int st = 0; st < NB && st < 2; ++st) off += ((u >> (NB - 1 - st)) & 1) ? (2 >> st) : 0;
    constexpr int NCH = (NB >= 2) ? 1 : (4 >> NB);
    const bool writer = (NB <= 2) || ((u & 1) == 0);
    merge(mua, za, acca);
    merge(mub, zb, accb);
    if (va) store_message_f16<NC, NCH>(A, ia, C, za, acca, cb + off, writer, lane);
    if (vb) store_message_f16<NC, NCH>(A, ib, C, zb, accb, cb + off, writer, lane);
}

template <int L>
static hipError_t launch_attn_pair_l(const AttnArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.n + 7) / 8)), block(256);
    switch (a.H) {
    case 4: attn_pair_kernel<L, 4><<<grid, block, 0, stream>>>(a); break;
    case 8: attn_pair_kernel<L, 8><<<grid, block, 0, stream>>>(a); break;
    case 16: attn_pair_kernel<L, 16><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attn_pair(int L, const AttnArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    if (a.n >= attn_pair_max_atoms(L, 8 * a.H)) return hipErrorInvalidValue;
    switch (L) {
    case 0: return launch_attn_pair_l<0>(a, stream);
    case 1: return launch_attn_pair_l<1>(a, stream);
    case 2: return launch_attn_pair_l<2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace e2v2
