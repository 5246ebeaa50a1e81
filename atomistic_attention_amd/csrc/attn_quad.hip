// Streaming neighbour attention, four targets per wave, with the weighted sums on
// the matrix cores (16-bit storage, l_max <= 2, 16 heads of 8 channels).
//
// E2Former-V2 explainer, section 3.1 (the message m_i = sum_j alpha_ij h'_j is
// formed on the fly) and section 3.2 (Algorithm 1: online softmax with a running
// maximum and normaliser, rows streamed once per pass, accumulation on chip,
// padded neighbours skipped).  The distance bias -- distance, Gaussian expansion,
// cosine envelope with its cutoff mask -- is computed in the kernel and never
// written out (FlashSchNet page, sections 2.1-2.2); each target's output row is
// written by one wave, with no atomics (section 2.3).
//
// A wave takes the four targets at processing slots 4 w .. 4 w + 3 (spatially
// close when the order comes from the cell list) and streams the union of their
// four lists, four entries at a time.  Per head, the four targets' messages are a
// small matrix product: (4 targets x 4 entries of softmax weights) times (4
// entries x the head's 8 channels of every component).  v_mfma_f32_4x4x4_16b_f16
// runs 16 independent 4x4x4 products, so block h of the instruction is head h:
// lane 4 h + t holds target t's weights (B operand) and receives target t's sums,
// lane 4 h + c holds value column c of the 4 entries (A operand), and 2 NC
// instructions cover the head's NC x 8 values.  The weights enter as an fp16 pair
// (hi + lo, about 2^-22 relative), the values are the stored fp16 h'.
// The logits q_t . k_j are 8-term fp32 dot products per head, eight
// v_mfma_f32_4x4x1_16b_f32 (block h; rows the entries, columns the targets), so
// the keys stay fp32.  The bias of the 16 (target, entry) pairs is one
// v_mfma_f32_16x16x32_f16 (Gaussians times log2(e) W_rbf), moved into the lanes of
// the logits by four ds_bpermute.
//
// The projection kernel writes h' rows in the layout loaded here
// (hp_quad_offset): lane 4 h + c takes, per component e, the dword
// (h'[e][8 h + c], h'[e][8 h + 4 + c]); each lane's first 4 floor(NC / 4) dwords
// sit together (16-byte loads), the rest in a tail region.  The A operand of an
// instruction is then two v_perm_b32 of the four entries' dwords.
//
// Softmax weights carry the row scale s_j of the stored h'_j (a power of two):
// a_j = exp2(l_j + log2 s_j - mu), with mu the running maximum of l_j + log2 s_j,
// raised only when it grows by more than 8 (so a_j <= 2^8 and the accumulators
// are rescaled rarely).  The normaliser sums exp2(l_j + zeta - mu) =
// a_j 2^(zeta - log2 s_j) for one fixed zeta per wave (the first entry's
// log2 s), and m = acc 2^zeta / z: both stay far from the fp32 limits unless the
// row scales of one union differ by more than about 2^100.
//
// The union: the four lists go to the four 16-lane rows of the wave as keys
// (j << 2) | list, rows 0 and 2 ascending and rows 1 and 3 descending; lists
// given in ascending order then need the last two bitonic merge phases only, any
// other order (the neighbour builder's scan order) the full sort.  Equal atoms
// fold into one entry (j << 4) | (bit mask of the lists holding it), compacted
// into LDS in atom order.  A list longer than 256 entries, or an atom listed
// twice in one list, sends the wave down the general path: the four lists
// streamed one after the other, each entry feeding its own target (an atom
// listed twice counts twice, as in the per-target kernel).
#include "attn_common.h"

#include <climits>

namespace e2v2 {

namespace {

constexpr int kQuadUnionMax = 1024;           // 4 lists of up to 256 entries

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void quad_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int sel4(const int (&v)[4], int i)
{
    return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// The union of the four lists into su (entries (j << 4) | mask, atom order,
// followed by 8 to 11 padding entries fill << 4: a valid row that no target
// uses); returns the entry count, or -1 when a list holds an atom twice.  sk is
// scratch for 64 E keys.  Every list must hold at most 16 E entries.
template <int E>
__device__ __forceinline__ int quad_union(const int32_t *__restrict__ idx, int n, const int (&st)[4],
                                          const int (&ln)[4], int fill, int *sk, int *su, int lane)
{
    constexpr int N = 64 * E, S = 16 * E;
    const int sg = lane >> 4;                       // list of this 16-lane row
    const int sst = sel4(st, sg), sln = sel4(ln, sg);
    const bool desc = (sg & 1) != 0;
    int key[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int p = (lane & 15) * E + k;          // position in the row's run
        const int x = desc ? S - 1 - p : p;         // entry of the list
        int kv = INT_MAX;
        if (x < sln) {
            const int j = idx[sst + x];
            if (j >= 0 && j < n) kv = (j << 2) | sg;
        }
        key[k] = kv;
    }
    const int nxt0 = __shfl_down(key[0], 1, 64);
    bool bad = false;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (k == E - 1 && (lane & 15) == 15) continue;   // end of the run
        const int nx = k < E - 1 ? key[k + 1] : nxt0;
        bad |= desc ? key[k] < nx : key[k] > nx;
    }
    if (__builtin_amdgcn_ballot_w64(bad) == 0) wave_bitonic_sort<E, 2 * S>(key, lane);
    else wave_bitonic_sort<E>(key, lane);
#pragma unroll
    for (int k = 0; k < E; ++k) sk[lane * E + k] = key[k];
    quad_lds_sync();
    int base = 0;
    bool dup = false;
#pragma unroll
    for (int m = 0; m < E; ++m) {
        const int x = m * 64 + lane;
        const int kv = sk[x];
        const int pv = x > 0 ? sk[x - 1] : -1;
        const bool live = kv != INT_MAX;
        const bool head = live && (pv >> 2) != (kv >> 2);
        dup |= live && pv == kv;
        int mask = 0;
        if (head) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                if (x + d < N) {
                    const int k2 = sk[x + d];
                    if (k2 != INT_MAX && (k2 >> 2) == (kv >> 2)) mask |= 1 << (k2 & 3);
                }
            }
        }
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(head);
        const int below = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
        if (head) su[base + below] = ((kv >> 2) << 4) | mask;
        base += __builtin_popcountll(bal);
    }
    if (__builtin_amdgcn_ballot_w64(dup) != 0) return -1;
    const int padn = ((base + 3) & ~3) + 8 - base;  // two groups of padding past the last
    if (lane < padn) su[base + lane] = fill << 4;
    quad_lds_sync();
    return base;
}

// One group's h' dwords of the four entries.
template <int NV, int NT> struct QuadRows {
    uint4 v[4][NV > 0 ? NV : 1];
    uint32_t tl[4][NT > 0 ? NT : 1];
};
// This lane's key piece and the position of the entry that lanes with the same
// (lane & 3) use (single-buffered: reloaded once the logits have used them).
struct QuadKeys {
    float4 k0, k1, pj;
};

}  // namespace

// Rows are addressed by 32-bit byte offsets (h' rows of 256 NC bytes, key rows of
// 512) and entry codes need n < 2^27.
long long attn_quad_max_atoms(int L)
{
    const long long row = 256LL * (L + 1) * (L + 1) > 512 ? 256LL * (L + 1) * (L + 1) : 512;
    const long long lim = (1LL << 32) / row;
    return lim < (1LL << 27) ? lim : (1LL << 27);
}

// The four targets at processing slots s0 .. s0 + 3, by one wave.
template <int L>
__device__ __forceinline__ void quad_body(const AttnArgs &A, long long s0, const _Float16 (*sWh)[64][8], int *sk,
                                          int *su, float4 *sq)
{
    constexpr int NC = n_comp(L);
    constexpr int C = 128;
    constexpr int D1 = 4 * (NC / 4);     // dwords per lane and row in the main region
    constexpr int D2 = NC - D1;          // and in the tail region
    constexpr int NV = D1 / 4;           // 16-byte loads per lane and row
    static_assert(D2 <= 1, "tail of one dword (NC = 1, 4, 9)");
    constexpr float LOG2E = 1.4426950408889634f;

    const int lane = threadIdx.x & 63;
    const int h = lane >> 2, t = lane & 3;      // head; target (B operand, sums) or column / entry (A operands)
    const int kq = lane >> 4, pm = lane & 15;   // bias product: Gaussian group; pair (target pm >> 2, entry pm & 3)
    const int R = A.R;
    const int n = A.n;
    if (s0 >= n) return;
    // ---- the four targets and their lists
    int my_i = -1, my_st = 0, my_ln = 0;
    if (lane < 4 && s0 + lane < n) {
        const int i = A.order ? A.order[s0 + lane] : (int)(s0 + lane);
        if (i >= 0 && i < n) {
            my_i = i;
            my_st = A.nbr_start[i];
            const int l0 = A.nbr_len[i];
            my_ln = l0 > 0 ? l0 : 0;
        }
    }
    int ti[4], st[4], ln[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        ti[q] = __builtin_amdgcn_readlane(my_i, q);
        st[q] = __builtin_amdgcn_readlane(my_st, q);
        ln[q] = __builtin_amdgcn_readlane(my_ln, q);
    }
    const int ifill = ti[0] >= 0 ? ti[0] : ti[1] >= 0 ? ti[1] : ti[2] >= 0 ? ti[2] : ti[3];
    if (ifill < 0) return;
    const int maxln = max(max(ln[0], ln[1]), max(ln[2], ln[3]));

    // ---- the stream: the union of the lists, or the lists one after the other
    int nu = -1;
    if (maxln <= 16) nu = quad_union<1>(A.nbr_idx, n, st, ln, ifill, sk, su, lane);
    else if (maxln <= 32) nu = quad_union<2>(A.nbr_idx, n, st, ln, ifill, sk, su, lane);
    else if (maxln <= 64) nu = quad_union<4>(A.nbr_idx, n, st, ln, ifill, sk, su, lane);
    else if (maxln <= 128) nu = quad_union<8>(A.nbr_idx, n, st, ln, ifill, sk, su, lane);
    else if (maxln <= 256) nu = quad_union<16>(A.nbr_idx, n, st, ln, ifill, sk, su, lane);
    nu = __builtin_amdgcn_readfirstlane(nu);
    const bool uni = nu >= 0;
    const long long tot64 = (long long)ln[0] + ln[1] + ln[2] + ln[3];
    const int tot = uni ? nu : (int)(tot64 < INT_MAX - 8 ? tot64 : INT_MAX - 8);
    const int G = (tot + 3) >> 2;
    // entry x of the sequential stream; past the end, or an index out of range, the
    // fill row with no target
    auto seq_code = [&](int x) -> int {
        if (x >= tot) return ifill << 4;
        int q = 0, off = x;
        if (off >= ln[0]) {
            off -= ln[0];
            q = 1;
            if (off >= ln[1]) {
                off -= ln[1];
                q = 2;
                if (off >= ln[2]) {
                    off -= ln[2];
                    q = 3;
                }
            }
        }
        const int j = A.nbr_idx[sel4(st, q) + off];
        return (j >= 0 && j < n) ? (j << 4) | (1 << q) : ifill << 4;
    };
    // codes of group g (wave-uniform); g may be G or G + 1 (padding only)
    auto codes = [&](int g, int (&cd)[4]) {
        if (uni) {
            const int4 v = *reinterpret_cast<const int4 *>(su + 4 * g);
            cd[0] = __builtin_amdgcn_readfirstlane(v.x);
            cd[1] = __builtin_amdgcn_readfirstlane(v.y);
            cd[2] = __builtin_amdgcn_readfirstlane(v.z);
            cd[3] = __builtin_amdgcn_readfirstlane(v.w);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) cd[r] = seq_code(4 * g + r);
        }
    };
    // code cd[t] in lane 4 h + t: three selects under constant lane masks
    auto lane_code = [&](const int (&cd)[4]) -> int {
        int v = cd[0];
        v = __builtin_amdgcn_inverse_ballot_w64(0x2222222222222222ull) ? cd[1] : v;
        v = __builtin_amdgcn_inverse_ballot_w64(0x4444444444444444ull) ? cd[2] : v;
        v = __builtin_amdgcn_inverse_ballot_w64(0x8888888888888888ull) ? cd[3] : v;
        return v;
    };

    // ---- per-lane constants
    const float qscale = LOG2E * 0.35355339059327373f;   // log2(e) / sqrt(8)
    // q of target t, head h, times qscale, parked in LDS (sq[2 lane], sq[2 lane + 1])
    // and read back per group as the B operands of the logit product
    {
        const int it = sel4(ti, t);
        const float *qr = A.q + (size_t)(it >= 0 ? it : ifill) * C + 8 * h;
        const float4 a = *reinterpret_cast<const float4 *>(qr), b = *reinterpret_cast<const float4 *>(qr + 4);
        const float s = it >= 0 ? qscale : 0.f;
        sq[2 * lane] = make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
        sq[2 * lane + 1] = make_float4(b.x * s, b.y * s, b.z * s, b.w * s);
    }
    float4 pt;                                            // target of bias pair pm
    {
        const int it = sel4(ti, pm >> 2);
        pt = A.pos4[it >= 0 ? it : ifill];
    }
    // Gaussians in the log2 domain: exp(-u^2 / 2) = exp2(-(g u)^2) with g^2 = log2(e) / 2,
    // u = (d - mu_k) / Delta; the envelope joins the exponent as log2(fc).
    const float gsc = 0.84932180028801904f;              // sqrt(log2(e) / 2)
    const float inv_delta = gsc * (float)(R - 1) / A.cutoff;
    const float cos_scale = 0.5f / A.cutoff;             // cos(pi d / rc) = cos(2 pi * d / (2 rc))
    const int bsrc = 4 * (16 * t + h);                   // lane of the bias product holding (target t, head h)

    floatx4 acc[NC][2];
#pragma unroll
    for (int e = 0; e < NC; ++e) acc[e][0] = acc[e][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mu = -1e30f, z = 0.f;
    int zeta = 0;

    auto rows_of = [&](const int (&cd)[4], int (&row)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) row[r] = cd[r] >> 4;
    };
    // Raw buffer loads: the row offset is a scalar, the lane's offset a constant
    // register, so a row costs no vector address arithmetic.
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(A.hp), 0,
                                                                        (int)(n * (256u * NC)), 0x00020000);
    const int vo0 = lane * (4 * D1), vot = 256 * D1 + lane * 4;
    auto issue_v = [&](QuadRows<NV, D2> &b, const int (&cd)[4]) {
        int row[4];
        rows_of(cd, row);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int so = (int)(uint32_t(row[r]) * uint32_t(256 * NC));   // < 2^32 (attn_quad_max_atoms)
#pragma unroll
            for (int v = 0; v < NV; ++v)
                b.v[r][v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(hrs, vo0 + 16 * v, so, 0));
            if constexpr (D2 > 0) b.tl[r][0] = __builtin_amdgcn_raw_buffer_load_b32(hrs, vot, so, 0);
        }
    };
    auto issue_k = [&](QuadKeys &kb, const int (&cd)[4]) {
        const int rk = lane_code(cd) >> 4;
        const unsigned char *kr = reinterpret_cast<const unsigned char *>(A.k) + (uint32_t(rk) * 512u + uint32_t(32 * h));
        kb.k0 = *reinterpret_cast<const float4 *>(kr);
        kb.k1 = *reinterpret_cast<const float4 *>(kr + 16);
        // positions: lanes 0..15 only (their distances are shared with the other rows)
        if (lane < 16)
            kb.pj = *reinterpret_cast<const float4 *>(reinterpret_cast<const unsigned char *>(A.pos4) + uint32_t(rk) * 16u);
    };

    // Masked scores (logit + bias + log2 s_r, base 2) of one group and its rows'
    // log2 scales; requests the next group's keys once this group's are read.
    auto scores = [&](QuadKeys &kb, const int (&cd)[4], const int (&cn)[4], bool first, float (&sc)[4],
                      int (&lsi)[4]) {
        // log2 of the four rows' scales (lanes 0..3 loaded rows 0..3), exact integers
#pragma unroll
        for (int r = 0; r < 4; ++r) lsi[r] = (int)((__builtin_amdgcn_readlane(__float_as_uint(kb.pj.w), r) >> 23) & 255u) - 127;
        if (first) zeta = lsi[0];
        // logits q_t . k_r of head h: lane 4 h + t, register r (two chains of four)
        const float4 qa = sq[2 * lane], qb = sq[2 * lane + 1];
        floatx4 S = {0.f, 0.f, 0.f, 0.f}, S2 = {0.f, 0.f, 0.f, 0.f};
        S = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k0.x, qa.x, S, 0, 0, 0);
        S2 = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k1.x, qb.x, S2, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k0.y, qa.y, S, 0, 0, 0);
        S2 = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k1.y, qb.y, S2, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k0.z, qa.z, S, 0, 0, 0);
        S2 = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k1.z, qb.z, S2, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k0.w, qa.w, S, 0, 0, 0);
        S2 = __builtin_amdgcn_mfma_f32_4x4x1f32(kb.k1.w, qb.w, S2, 0, 0, 0);
        S += S2;
        // bias of pair pm (target pm >> 2, entry pm & 3 = this lane's row), also for
        // pairs that the mask drops below (their logits never enter)
        floatx4 bias;
        {
            const float dx = kb.pj.x - pt.x, dy = kb.pj.y - pt.y, dz = kb.pj.z - pt.z;
            const float dl = __builtin_amdgcn_sqrtf(dx * dx + dy * dy + dz * dz);   // v_sqrt_f32, 1 ulp; lanes 0..15
            const float d = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * pm, __float_as_int(dl)));
            const float fc = d < A.cutoff ? 0.5f * (__builtin_amdgcn_cosf(d * cos_scale) + 1.f) : 0.f;   // cutoff mask
            const float lfc = __builtin_amdgcn_logf(fmaxf(fc, 0.f));   // log2; fc = 0 gives -inf, phi = 0
            // past the cutoff phi is 0 whatever u is; the clamp keeps the ratio q below finite
            const float t0 = fmaf(fminf(d, A.cutoff), inv_delta, -gsc * (float)(8 * kq));
            // kb is read: request the next group's keys and positions into it
            __builtin_amdgcn_sched_barrier(0);
            issue_k(kb, cn);
            __builtin_amdgcn_sched_barrier(0);
            // A operand: lane (kq, pm) holds phi_k of pair pm for k = 8 kq + i (+ 32).
            // With u_i = u - g i (g = gsc), phi_{i+1} / phi_i = exp2(2 g u - g^2) e^{-i}: two
            // exponentials and a product chain give the lane's 8 consecutive Gaussians.
            auto group = [&](int g, floatx4 ac) {
                const float u = t0 - gsc * (float)(32 * g);
                float phi = __builtin_amdgcn_exp2f(fmaf(-u, u, lfc));
                float q = __builtin_amdgcn_exp2f(fmaf(2.f * gsc, u, -gsc * gsc));
                half8_t a;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a[i] = (_Float16)phi;
                    phi *= q;
                    q *= 0.36787944117144233f;                      // exp2(-2 g^2) = 1 / e
                }
                const half8_t w = *reinterpret_cast<const half8_t *>(&sWh[g][lane][0]);
                return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, w, ac, 0, 0, 0);
            };
            bias = group(0, floatx4{0.f, 0.f, 0.f, 0.f});
            if (R > 32) bias = group(1, bias);
        }
        // lane (kq', pm') of the product holds pairs 4 kq' + i (target kq', entry i) of
        // head pm': move target t, head h to lane 4 h + t
        float br[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) br[r] = __int_as_float(__builtin_amdgcn_ds_bpermute(bsrc, __float_as_int(bias[r])));
        // entry r feeds the targets in bits 0..3 of its code: as a lane mask, the
        // lanes 4 h + t of those targets
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t m32 = uint32_t(cd[r] & 15) * 0x11111111u;
            const bool on = __builtin_amdgcn_inverse_ballot_w64((uint64_t(m32) << 32) | m32);
            sc[r] = on ? S[r] + br[r] + (float)lsi[r] : -INFINITY;
        }
    };
    // The lazily raised running maximum, then the group's weights as fp16 pairs.
    auto finish = [&](const float (&sc)[4], const int (&lsi)[4], half4_t &bh, half4_t &bl) {
        const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        const bool grow = mx > mu + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float mun = grow ? mx : mu;
            const float corr = __builtin_amdgcn_exp2f(mu - mun);
            z *= corr;
#pragma unroll
            for (int e = 0; e < NC; ++e)
#pragma unroll
                for (int f = 0; f < 2; ++f) acc[e][f] *= corr;
            mu = mun;
        }
        // z gains a 2^(zeta - log2 s_r): a product with a power of two built from
        // its exponent field (clamped to the normal range), exact like ldexp
        float a[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            a[r] = __builtin_amdgcn_exp2f(sc[r] - mu);
            const int ex = min(max(zeta - lsi[r] + 127, 1), 254);
            z = fmaf(a[r], __uint_as_float(uint32_t(ex) << 23), z);
        }
        const half4_t hv = __builtin_convertvector(*reinterpret_cast<const floatx4 *>(a), half4_t);
        const floatx4 hf = __builtin_convertvector(hv, floatx4);
        bh = hv;
        bl = __builtin_convertvector(*reinterpret_cast<const floatx4 *>(a) - hf, half4_t);
    };
    // The group's weighted sum into the accumulators.
    auto sums = [&](const QuadRows<NV, D2> &b, const half4_t &bh, const half4_t &bl) {
        // weighted sum: A operand of (component e, channel half f) from the four rows'
        // dword e, low halves (f = 0) or high halves (f = 1)
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            uint32_t w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (e < D1) {
                    const uint4 &v = b.v[r][e >> 2];
                    const int c = e & 3;
                    w[r] = c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
                } else {
                    w[r] = b.tl[r][0];
                }
            }
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const uint32_t sel = f ? 0x07060302u : 0x05040100u;
                const uint32_t a01 = __builtin_amdgcn_perm(w[1], w[0], sel);
                const uint32_t a23 = __builtin_amdgcn_perm(w[3], w[2], sel);
                const half4_t av = __builtin_bit_cast(half4_t, make_uint2(a01, a23));
                acc[e][f] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, bh, acc[e][f], 0, 0, 0);
                acc[e][f] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, bl, acc[e][f], 0, 0, 0);
            }
        }
    };

    // ---- the stream.  The next group's keys and positions are requested as soon as
    //      this group's logits and distances have read them, its rows as soon as
    //      this group's sums have used the row buffer; the group after the last reads
    //      the fill row.
    QuadRows<NV, D2> b;
    QuadKeys kb;
    kb.pj = make_float4(0.f, 0.f, 0.f, 0.f);
    int c0[4], c1[4];
    codes(0, c0);
    __builtin_amdgcn_sched_barrier(0);
    issue_k(kb, c0);
    __builtin_amdgcn_sched_barrier(0);
    issue_v(b, c0);
    __builtin_amdgcn_sched_barrier(0);
    for (int g = 0; g < G; ++g) {
        codes(g + 1, c1);
        half4_t bh, bl;
        float sc[4];
        int lsi[4];
        scores(kb, c0, c1, g == 0, sc, lsi);
        finish(sc, lsi, bh, bl);
        sums(b, bh, bl);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(b, c1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 4; ++r) c0[r] = c1[r];
    }

    // ---- m_t = acc 2^zeta / z per head; one power-of-two scale per target (the
    //      largest |m_t| below 2^14 s, as for the source features), fp16 store
    const int it = sel4(ti, t);
    const float f = z > 0.f ? __builtin_ldexpf(1.f / z, zeta) : 0.f;
    unsigned mb = 0u;
#pragma unroll
    for (int e = 0; e < NC; ++e)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int c = 0; c < 4; ++c) mb = max(mb, __float_as_uint(acc[e][g][c] * f) & 0x7fffffffu);
#pragma unroll
    for (int d = 4; d <= 32; d <<= 1) mb = max(mb, (unsigned)__shfl_xor((int)mb, d, 64));
    unsigned sb = 127u;                                  // scale 1 for zero or non-finite rows
    if (mb != 0u && mb < 0x7f800000u) {
        const unsigned bx = mb >> 23;
        sb = bx > 13u ? bx - 13u : 1u;
    }
    const float scm = __uint_as_float(sb << 23), inv = __uint_as_float((254u - sb) << 23);
    if (it < 0) return;
    if (h == 0) A.msc[it] = scm;
#pragma unroll
    for (int e = 0; e < NC; ++e) {
        const size_t o = ((size_t)it * NC + e) * C + 8 * h;
        _Float16 hv[8];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int c = 0; c < 4; ++c) hv[4 * g + c] = (_Float16)(acc[e][g][c] * f * inv);
        uint4 pk;
        pk.x = uint32_t(__builtin_bit_cast(uint16_t, hv[0])) | (uint32_t(__builtin_bit_cast(uint16_t, hv[1])) << 16);
        pk.y = uint32_t(__builtin_bit_cast(uint16_t, hv[2])) | (uint32_t(__builtin_bit_cast(uint16_t, hv[3])) << 16);
        pk.z = uint32_t(__builtin_bit_cast(uint16_t, hv[4])) | (uint32_t(__builtin_bit_cast(uint16_t, hv[5])) << 16);
        pk.w = uint32_t(__builtin_bit_cast(uint16_t, hv[6])) | (uint32_t(__builtin_bit_cast(uint16_t, hv[7])) << 16);
        *reinterpret_cast<uint4 *>(A.mh + o) = pk;
        if (A.m_tap) {
            float *mt = A.m_tap + o;
            *reinterpret_cast<float4 *>(mt) = make_float4((float)hv[0] * scm, (float)hv[1] * scm, (float)hv[2] * scm, (float)hv[3] * scm);
            *reinterpret_cast<float4 *>(mt + 4) = make_float4((float)hv[4] * scm, (float)hv[5] * scm, (float)hv[6] * scm, (float)hv[7] * scm);
        }
    }
}

template <int L>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void attn_quad_kernel(const AttnArgs A)
{
    const int wv = threadIdx.x >> 6;
    // B operand of the bias product in fp16, log2(e) W_rbf[k][head] zero-padded to
    // 64 x 16, as v_mfma_f32_16x16x32_f16 fragments: group g, lane l holds
    // k = 32 g + 8 (l / 16) + i (i < 8) for head column l % 16.
    __shared__ __align__(16) _Float16 sWh[2][64][8];
    __shared__ int sK[4][kQuadUnionMax];
    __shared__ __align__(16) int sU[4][kQuadUnionMax + 12];
    __shared__ float4 sQ[4][128];
    for (int e = threadIdx.x; e < 2 * 64 * 8; e += 256) {
        const int g = e >> 9, l = (e >> 3) & 63, i = e & 7;
        const int k = 32 * g + 8 * (l >> 4) + i;
        sWh[g][l][i] = (_Float16)((k < A.R) ? A.w_rbf[k * 16 + (l & 15)] * 1.4426950408889634f : 0.f);
    }
    __syncthreads();
    // Workgroups go to the 8 XCDs round robin; each XCD gets one contiguous run of
    // target quads, so the targets one XCD works on at a time are close together
    // and share rows in its L2.
    const int nb = gridDim.x, xcd = blockIdx.x & 7, kth = blockIdx.x >> 3;
    const int lb = xcd * (nb >> 3) + (xcd < (nb & 7) ? xcd : (nb & 7)) + kth;
    const int ps = __builtin_amdgcn_readfirstlane(lb * 4 + wv);
    quad_body<L>(A, 4LL * ps, sWh, sK[wv], sU[wv], sQ[wv]);
}


hipError_t launch_attn_quad(int L, const AttnArgs &a, hipStream_t stream)
{
    if (a.n <= 0) return hipSuccess;
    if (a.H != 16 || a.C != 128 || a.n >= attn_quad_max_atoms(L)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.n + 15) / 16)), block(256);
    switch (L) {
    case 0: attn_quad_kernel<0><<<grid, block, 0, stream>>>(a); break;
    case 1: attn_quad_kernel<1><<<grid, block, 0, stream>>>(a); break;
    case 2: attn_quad_kernel<2><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace e2v2
