// Compile-time enumeration of the terms of the exact edge-equivalent form
// evaluated node by node (E2Former-V2 explainer, section 1.2: Wigner-6j
// recoupling).  The host fills the values in the same order (e2v2_api.cpp), the
// kernels (edge.hip) unroll the same lists, so every index is static.
//
// With an origin o, x_j = (r_j - o) / r_c and y_i = (o - r_i) / r_c, the edge
// vector is x_j + y_i.  The solid harmonic of a sum splits (addition theorem)
//   S^lf(x + y) = sum_lam a(lf, lam) (S^lam(x) (x) S^mu(y))^lf,  mu = lf - lam,
// and the coupling of v with that pair recouples (6j):
//   (v^li (x) (S^lam (x) S^mu)^lf)^lo = sum_lp U (( v^li (x) S^lam )^lp (x) S^mu)^lo.
// So source j carries blocks G^(li, lam, lp) = (v_j^li (x) S^lam(x_j))^lp, the
// stream sums alpha_ij G_j, and target i couples the sum with S^mu(y_i).
#pragma once

#include "e2v2_internal.h"

namespace e2v2 {
namespace edge {

constexpr int kMaxEdgeL = 2;

__host__ __device__ constexpr int iabs(int a) { return a < 0 ? -a : a; }

// Real-basis selection rule of T[m_a, m_b, m_c] for the triple (la, lb, lc): in the
// complex basis m_c = m_a + m_b, so |m_c| is |m_a| + |m_b| or ||m_a| - |m_b||, and
// the number of sine-type (m < 0) factors has the parity of la + lb + lc.  Every
// nonzero entry satisfies it (the host checks this while filling the values).
__host__ __device__ constexpr bool real_allowed(int la, int lb, int lc, int ma, int mb, int mc)
{
    const int a = iabs(ma), b = iabs(mb), c = iabs(mc);
    if (c != a + b && c != iabs(a - b)) return false;
    return (((ma < 0) ^ (mb < 0) ^ (mc < 0)) ? 1 : 0) == ((la + lb + lc) & 1);
}

// Block (li, lam, lp) of the source features is kept when some path (li, lf, lo)
// with lf >= lam reaches lo from lp through mu = lf - lam.
template <int L>
__host__ __device__ constexpr bool block_used(int li, int lam, int lp)
{
    if (!is_path(li, lam, lp)) return false;
    for (int lf = lam; lf <= L; ++lf)
        for (int lo = 0; lo <= L; ++lo)
            if (is_path(li, lf, lo) && is_path(lp, lf - lam, lo)) return true;
    return false;
}

struct Block {
    int li, lam, lp, off;            // components off .. off + 2 lp
};
constexpr int kMaxBlocks = 48;
struct Blocks {
    int n, ncomp;
    Block b[kMaxBlocks];
};
template <int L>
constexpr Blocks blocks()
{
    Blocks r = {};
    int off = 0;
    for (int li = 0; li <= L; ++li)
        for (int lam = 0; lam <= L; ++lam)
            for (int lp = 0; lp <= li + lam; ++lp)
                if (block_used<L>(li, lam, lp)) {
                    r.b[r.n++] = Block{li, lam, lp, off};
                    off += 2 * lp + 1;
                }
    r.ncomp = off;
    return r;
}

// Source terms: G[eg] += T^(li, lam, lp)[mi, ml, mp] v[ei] S(x)[el].
struct SrcTerm {
    int ei, el, eg;
};
constexpr int kMaxSrcTerms = 256;
struct SrcTerms {
    int n;
    SrcTerm t[kMaxSrcTerms];
};
template <int L>
constexpr SrcTerms src_terms()
{
    constexpr Blocks B = blocks<L>();
    SrcTerms r = {};
    for (int k = 0; k < B.n; ++k) {
        const Block &b = B.b[k];
        for (int mi = -b.li; mi <= b.li; ++mi)
            for (int ml = -b.lam; ml <= b.lam; ++ml)
                for (int mp = -b.lp; mp <= b.lp; ++mp)
                    if (real_allowed(b.li, b.lam, b.lp, mi, ml, mp))
                        r.t[r.n++] = SrcTerm{b.li * b.li + b.li + mi, b.lam * b.lam + b.lam + ml, b.off + mp + b.lp};
    }
    return r;
}

// Target terms: out[eo] += w[p] a(lf, lam) U T^(lp, mu, lo)[mp, mu_m, mo] M[eg] S(y)[em]
// for path p = (li, lf, lo), lam <= lf, mu = lf - lam, block (li, lam, lp).
struct TgtTerm {
    int p, eg, em, eo;
};
constexpr int kMaxTgtTerms = 512;
struct TgtTerms {
    int n;
    TgtTerm t[kMaxTgtTerms];
};
template <int L>
constexpr TgtTerms tgt_terms()
{
    constexpr Blocks B = blocks<L>();
    TgtTerms r = {};
    int p = 0;
    for (int lo = 0; lo <= L; ++lo)
        for (int li = 0; li <= L; ++li)
            for (int lf = 0; lf <= L; ++lf) {
                if (!is_path(li, lf, lo)) continue;
                for (int lam = 0; lam <= lf; ++lam) {
                    const int mu = lf - lam;
                    for (int k = 0; k < B.n; ++k) {
                        const Block &b = B.b[k];
                        if (b.li != li || b.lam != lam || !is_path(b.lp, mu, lo)) continue;
                        for (int mp = -b.lp; mp <= b.lp; ++mp)
                            for (int mm = -mu; mm <= mu; ++mm)
                                for (int mo = -lo; mo <= lo; ++mo)
                                    if (real_allowed(b.lp, mu, lo, mp, mm, mo))
                                        r.t[r.n++] = TgtTerm{p, b.off + mp + b.lp, mu * mu + mu + mm, lo * lo + lo + mo};
                    }
                }
                ++p;
            }
    return r;
}

// Host values in the orders above (built once per process; nullptr for l_max > 2).
const float *src_values(int lmax);
const float *tgt_values(int lmax);

}  // namespace edge
}  // namespace e2v2
