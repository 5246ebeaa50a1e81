// Host side of the e2v2 C ABI: argument validation, workspace layout, kernel
// launches and the constant tables the kernels take by value.
//
// Tables (built once per process):
//  * EAAS coefficients.  In the frame whose z axis is the position vector the
//    encoding Y^{l_f}(z) is sqrt(2 l_f + 1) on m_f = 0 and zero elsewhere
//    (E2Former-V2 explainer, section 2.1), so path (l_i, l_f, l_o) reduces to
//    out_{m_o} = sqrt(2 l_f + 1) T[m_i, 0, m_o] x~_{m_i} with m_i = +-m_o
//    (section 2.2).  T is the real-basis Clebsch-Gordan tensor: complex
//    Condon-Shortley coefficients (Racah's closed formula) conjugated into the
//    real basis, real part for even l_i + l_f + l_o, imaginary part for odd.
//  * Wigner-D sampling: 2l+1 fixed directions X per l in {2, 3} and the inverse
//    of Y^l(X), so a kernel gets D^l(R) = Y^l(R X) Y^l(X)^{-1} from a handful of
//    harmonic evaluations.  The directions are picked from a Fibonacci sphere
//    to keep Y^l(X) well conditioned.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <complex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/e2v2.h"
#include "e2v2_internal.h"
#include "edge_terms.h"

namespace e2v2 {
namespace {

// ---------------------------------------------------------------- Clebsch-Gordan
double fact(int k)
{
    double r = 1.0;
    for (int i = 2; i <= k; ++i) r *= i;
    return r;
}

// <j1 m1; j2 m2 | J M>, Racah's formula (integer momenta, small enough for doubles).
double cg(int j1, int m1, int j2, int m2, int J, int M)
{
    if (m1 + m2 != M || std::abs(m1) > j1 || std::abs(m2) > j2 || std::abs(M) > J) return 0.0;
    if (J < std::abs(j1 - j2) || J > j1 + j2) return 0.0;
    const double pre = std::sqrt((2.0 * J + 1.0) * fact(J + j1 - j2) * fact(J - j1 + j2) * fact(j1 + j2 - J) /
                                 fact(j1 + j2 + J + 1) * fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) *
                                 fact(j2 - m2) * fact(j2 + m2));
    double sum = 0.0;
    for (int k = 0; k <= j1 + j2 + J; ++k) {
        const int a[6] = {k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k};
        bool ok = true;
        for (int v : a) ok = ok && v >= 0;
        if (!ok) continue;
        double den = 1.0;
        for (int v : a) den *= fact(v);
        sum += ((k & 1) ? -1.0 : 1.0) / den;
    }
    return pre * sum;
}

// Complex -> real basis: Y_real[m] = sum_mu U(m, mu) Y_complex[mu].
std::complex<double> U(int l, int m, int mu)
{
    const double r2 = 1.0 / std::sqrt(2.0);
    const double sgn = (std::abs(m) & 1) ? -1.0 : 1.0;
    if (m == 0) return mu == 0 ? 1.0 : 0.0;
    if (m > 0) {
        if (mu == -m) return r2;
        if (mu == m) return sgn * r2;
        return 0.0;
    }
    if (mu == m) return std::complex<double>(0.0, r2);
    if (mu == -m) return std::complex<double>(0.0, -sgn * r2);
    (void)l;
    return 0.0;
}

// sqrt(2 lf + 1) * T[m_i, m_f = 0, m_o] in the real basis.
double eaas_entry(int li, int lf, int lo, int mi, int mo)
{
    std::complex<double> acc = 0.0;
    for (int mu = -std::min(li, lo); mu <= std::min(li, lo); ++mu)   // m_f = 0 forces mu_i = mu_o
        acc += std::conj(U(li, mi, mu)) * U(lo, mo, mu) * cg(li, mu, lf, 0, lo, mu);
    const double v = ((li + lf + lo) & 1) ? acc.imag() : acc.real();
    return std::sqrt(2.0 * lf + 1.0) * v;
}

// ---------------------------------------------------------------- Wigner-D sampling
void sh_block(int l, const double *x, double *o)
{
    if (l == 2) sh_l2(x[0], x[1], x[2], o);
    else sh_l3(x[0], x[1], x[2], o);
}

// Gauss-Jordan inverse with partial pivoting; returns false if singular.
bool invert(int k, const double *A, double *Ainv)
{
    double M[7][14];
    for (int r = 0; r < k; ++r)
        for (int c = 0; c < 2 * k; ++c) M[r][c] = c < k ? A[r * k + c] : (c - k == r ? 1.0 : 0.0);
    for (int c = 0; c < k; ++c) {
        int piv = c;
        for (int r = c + 1; r < k; ++r)
            if (std::fabs(M[r][c]) > std::fabs(M[piv][c])) piv = r;
        if (std::fabs(M[piv][c]) < 1e-12) return false;
        for (int cc = 0; cc < 2 * k; ++cc) std::swap(M[c][cc], M[piv][cc]);
        const double d = M[c][c];
        for (int cc = 0; cc < 2 * k; ++cc) M[c][cc] /= d;
        for (int r = 0; r < k; ++r)
            if (r != c) {
                const double f = M[r][c];
                for (int cc = 0; cc < 2 * k; ++cc) M[r][cc] -= f * M[c][cc];
            }
    }
    for (int r = 0; r < k; ++r)
        for (int c = 0; c < k; ++c) Ainv[r * k + c] = M[r][c + k];
    return true;
}

// Pick 2l+1 directions with a well-conditioned Y^l(X) (Frobenius condition number).
void pick_samples(int l, double (*xs)[3], double *inv)
{
    const int k = 2 * l + 1;
    const int npts = 48;
    double pts[48][3];
    const double ga = M_PI * (3.0 - std::sqrt(5.0));
    for (int i = 0; i < npts; ++i) {
        const double z = 1.0 - (i + 0.5) * 2.0 / npts, r = std::sqrt(1.0 - z * z);
        pts[i][0] = r * std::cos(ga * i);
        pts[i][1] = r * std::sin(ga * i);
        pts[i][2] = z;
    }
    uint64_t s = 0x9E3779B97F4A7C15ull;
    double best = 1e300;
    int sel[7], bsel[7] = {0};
    for (int trial = 0; trial < 4000; ++trial) {
        for (int a = 0; a < k; ++a) {
            bool dup;
            do {
                s ^= s << 13; s ^= s >> 7; s ^= s << 17;
                sel[a] = (int)(s % npts);
                dup = false;
                for (int b = 0; b < a; ++b) dup = dup || sel[b] == sel[a];
            } while (dup);
        }
        double A[49], Ai[49];
        for (int c = 0; c < k; ++c) {       // A[m][s] = Y^l_m(x_s)
            double o[7];
            sh_block(l, pts[sel[c]], o);
            for (int m = 0; m < k; ++m) A[m * k + c] = o[m];
        }
        if (!invert(k, A, Ai)) continue;
        double na = 0, ni = 0;
        for (int e = 0; e < k * k; ++e) { na += A[e] * A[e]; ni += Ai[e] * Ai[e]; }
        const double cond = std::sqrt(na * ni);
        if (cond < best) {
            best = cond;
            std::copy(sel, sel + k, bsel);
            std::copy(Ai, Ai + k * k, inv);
        }
    }
    for (int a = 0; a < k; ++a)
        for (int d = 0; d < 3; ++d) xs[a][d] = pts[bsel[a]][d];
}

Tables g_tables;
std::once_flag g_once;

void build_tables()
{
    std::memset(&g_tables, 0, sizeof(g_tables));
    int p = 0;
    for (int lo = 0; lo <= kMaxL; ++lo)
        for (int li = 0; li <= kMaxL; ++li)
            for (int lf = 0; lf <= kMaxL; ++lf) {
                if (!is_path(li, lf, lo)) continue;
                const bool odd = (li + lf + lo) & 1;
                for (int mo = -lo; mo <= lo; ++mo) {
                    const int mi = odd ? -mo : mo;
                    if (std::abs(mi) > li) continue;
                    g_tables.eaas.c[p][mo + lo] = (float)eaas_entry(li, lf, lo, mi, mo);
                }
                ++p;
            }
    pick_samples(2, g_tables.ds.x2, &g_tables.ds.inv2[0][0]);
    pick_samples(3, g_tables.ds.x3, &g_tables.ds.inv3[0][0]);
}

// Path indices depend on lmax (l_o is the outer loop), so the table for a
// smaller lmax is the lmax = 3 table re-indexed.
void eaas_for_lmax(int lmax, EaasCoef &out)
{
    std::memset(&out, 0, sizeof(out));
    const Tables &t = host_tables();
    for (int lo = 0; lo <= lmax; ++lo)
        for (int li = 0; li <= lmax; ++li)
            for (int lf = 0; lf <= lmax; ++lf) {
                if (!is_path(li, lf, lo)) continue;
                const int src = path_index(kMaxL, li, lf, lo), dst = path_index(lmax, li, lf, lo);
                for (int e = 0; e < 2 * kMaxL + 1; ++e) out.c[dst][e] = t.eaas.c[src][e];
            }
}

EaasCoef g_by_lmax[kMaxL + 1];
std::once_flag g_once_l;

// Real-basis coupling tensor T[m_i, m_f, m_o] = sum conj(U_li) conj(U_lf) U_lo C(l_i mu_i; l_f mu_f | l_o mu_o),
// real part for even l_i + l_f + l_o, imaginary part for odd.
double coupling_entry(int li, int lf, int lo, int mi, int mf, int mo)
{
    std::complex<double> acc = 0.0;
    for (int a = -li; a <= li; ++a)
        for (int b = -lf; b <= lf; ++b) {
            const int M = a + b;
            if (std::abs(M) > lo) continue;
            acc += std::conj(U(li, mi, a)) * std::conj(U(lf, mf, b)) * U(lo, mo, M) * cg(li, a, lf, b, lo, M);
        }
    return ((li + lf + lo) & 1) ? acc.imag() : acc.real();
}

float g_yval[kMaxL + 1][kMaxYTerms];
std::once_flag g_once_yval;

template <int L>
void build_yval(float *out)
{
    constexpr YTerms T = ygrad_terms<L>();
    static_assert(T.n <= kMaxYTerms, "coupling entry table too small");
    for (int q = 0; q < T.n; ++q) {
        const YTerm &t = T.t[q];
        auto lm = [](int e, int &l, int &m) { l = 0; while ((l + 1) * (l + 1) <= e) ++l; m = e - l * l - l; };
        int li, mi, lf, mf, lo, mo;
        lm(t.ei, li, mi);
        lm(t.ef, lf, mf);
        lm(t.eo, lo, mo);
        out[q] = (float)coupling_entry(li, lf, lo, mi, mf, mo);
    }
}

}  // namespace

const float *ygrad_values(int lmax)
{
    std::call_once(g_once_yval, [] {
        std::memset(g_yval, 0, sizeof(g_yval));
        build_yval<1>(g_yval[1]);
        build_yval<2>(g_yval[2]);
        build_yval<3>(g_yval[3]);
    });
    return g_yval[lmax];
}

// ---------------------------------------------------------------- edge-form tables
namespace {
double binom(int a, int b)
{
    double r = 1.0;
    for (int k = 1; k <= b; ++k) r = r * (a - b + k) / k;
    return r;
}
// Addition theorem of the component-normalised solid harmonics:
// S^lf(x + y) = sum_lam a (S^lam(x) (x) S^(lf - lam)(y))^lf.
double addition_coef(int lf, int lam)
{
    const int mu = lf - lam;
    return std::sqrt(binom(2 * lf, 2 * lam) * (2.0 * lf + 1.0) / ((2.0 * lam + 1.0) * (2.0 * mu + 1.0)));
}
// 6j recoupling coefficients U(lp) in
//   (v^li (x) (a^lam (x) b^mu)^lf)^lo = sum_lp U(lp) ((v^li (x) a^lam)^lp (x) b^mu)^lo,
// from their definition as contractions of four coupling tensors: the left side
// and each term of the right side are 4-index tensors [m_i, m_lam, m_mu, m_o];
// U solves the least-squares fit of the left side by the right-side terms, which
// must be exact (residual below 1e-9 of the left side, else false).
bool recouple(int li, int lam, int mu, int lf, int lo, std::vector<int> &lps, std::vector<double> &U)
{
    const int ni = 2 * li + 1, na = 2 * lam + 1, nb = 2 * mu + 1, nf = 2 * lf + 1, no = 2 * lo + 1;
    const int sz = ni * na * nb * no;
    auto at = [&](int i, int a, int b, int o) { return ((i * na + a) * nb + b) * no + o; };
    std::vector<double> Lt(sz, 0.0);
    for (int i = 0; i < ni; ++i)
        for (int a = 0; a < na; ++a)
            for (int b = 0; b < nb; ++b)
                for (int o = 0; o < no; ++o) {
                    double acc = 0.0;
                    for (int f = 0; f < nf; ++f)
                        acc += coupling_entry(lam, mu, lf, a - lam, b - mu, f - lf) *
                               coupling_entry(li, lf, lo, i - li, f - lf, o - lo);
                    Lt[at(i, a, b, o)] = acc;
                }
    lps.clear();
    std::vector<std::vector<double>> Bs;
    for (int lp = std::abs(li - lam); lp <= li + lam; ++lp) {
        if (!is_path(lp, mu, lo)) continue;
        const int np = 2 * lp + 1;
        std::vector<double> B(sz, 0.0);
        for (int i = 0; i < ni; ++i)
            for (int a = 0; a < na; ++a)
                for (int b = 0; b < nb; ++b)
                    for (int o = 0; o < no; ++o) {
                        double acc = 0.0;
                        for (int m = 0; m < np; ++m)
                            acc += coupling_entry(li, lam, lp, i - li, a - lam, m - lp) *
                                   coupling_entry(lp, mu, lo, m - lp, b - mu, o - lo);
                        B[at(i, a, b, o)] = acc;
                    }
        lps.push_back(lp);
        Bs.push_back(B);
    }
    const int k = (int)lps.size();
    double Gm[8][9] = {};
    for (int r = 0; r < k; ++r) {
        for (int c = 0; c < k; ++c) {
            double g = 0.0;
            for (int e = 0; e < sz; ++e) g += Bs[r][e] * Bs[c][e];
            Gm[r][c] = g;
        }
        double rhs = 0.0;
        for (int e = 0; e < sz; ++e) rhs += Bs[r][e] * Lt[e];
        Gm[r][k] = rhs;
    }
    for (int c = 0; c < k; ++c) {                       // Gauss-Jordan on the Gram system
        int piv = c;
        for (int r = c + 1; r < k; ++r)
            if (std::fabs(Gm[r][c]) > std::fabs(Gm[piv][c])) piv = r;
        if (std::fabs(Gm[piv][c]) < 1e-14) return false;
        for (int cc = 0; cc <= k; ++cc) std::swap(Gm[c][cc], Gm[piv][cc]);
        for (int r = 0; r < k; ++r)
            if (r != c) {
                const double f = Gm[r][c] / Gm[c][c];
                for (int cc = 0; cc <= k; ++cc) Gm[r][cc] -= f * Gm[c][cc];
            }
    }
    U.assign(k, 0.0);
    for (int r = 0; r < k; ++r) U[r] = Gm[r][k] / Gm[r][r];
    double res = 0.0, nrm = 0.0;
    for (int e = 0; e < sz; ++e) {
        double fit = 0.0;
        for (int r = 0; r < k; ++r) fit += U[r] * Bs[r][e];
        res += (Lt[e] - fit) * (Lt[e] - fit);
        nrm += Lt[e] * Lt[e];
    }
    return res <= 1e-18 * std::max(nrm, 1e-300) || nrm == 0.0;
}

struct EdgeTables {
    bool ok[edge::kMaxEdgeL + 1];
    double src[edge::kMaxEdgeL + 1][edge::kMaxSrcTerms];
    double tgt[edge::kMaxEdgeL + 1][edge::kMaxTgtTerms];
    float srcf[edge::kMaxEdgeL + 1][edge::kMaxSrcTerms];
    float tgtf[edge::kMaxEdgeL + 1][edge::kMaxTgtTerms];
};
EdgeTables g_edge;
std::once_flag g_once_edge;

void comp_lm(int e, int &l, int &m)
{
    l = 0;
    while ((l + 1) * (l + 1) <= e) ++l;
    m = e - l * l - l;
}

template <int L>
bool build_edge(double *src, double *tgt)
{
    constexpr edge::Blocks B = edge::blocks<L>();
    constexpr edge::SrcTerms S = edge::src_terms<L>();
    constexpr edge::TgtTerms T = edge::tgt_terms<L>();
    static_assert(B.n <= edge::kMaxBlocks && S.n <= edge::kMaxSrcTerms && T.n <= edge::kMaxTgtTerms, "edge tables");
    auto block_of = [&](int eg) -> const edge::Block & {
        int k = 0;
        while (!(eg >= B.b[k].off && eg < B.b[k].off + 2 * B.b[k].lp + 1)) ++k;
        return B.b[k];
    };
    // every nonzero coupling entry of a used block or a target triple obeys the selection rule
    for (int k = 0; k < B.n; ++k) {
        const edge::Block &b = B.b[k];
        for (int mi = -b.li; mi <= b.li; ++mi)
            for (int ml = -b.lam; ml <= b.lam; ++ml)
                for (int mp = -b.lp; mp <= b.lp; ++mp)
                    if (!edge::real_allowed(b.li, b.lam, b.lp, mi, ml, mp) &&
                        std::fabs(coupling_entry(b.li, b.lam, b.lp, mi, ml, mp)) > 1e-12)
                        return false;
    }
    for (int q = 0; q < S.n; ++q) {
        const edge::SrcTerm &t = S.t[q];
        int li, mi, lam, ml;
        comp_lm(t.ei, li, mi);
        comp_lm(t.el, lam, ml);
        const edge::Block &b = block_of(t.eg);
        src[q] = coupling_entry(li, lam, b.lp, mi, ml, t.eg - b.off - b.lp);
    }
    int paths[64][3], np = 0;
    for (int lo = 0; lo <= L; ++lo)
        for (int li = 0; li <= L; ++li)
            for (int lf = 0; lf <= L; ++lf)
                if (is_path(li, lf, lo)) {
                    paths[np][0] = li; paths[np][1] = lf; paths[np][2] = lo;
                    ++np;
                }
    std::vector<int> lps;
    std::vector<double> U;
    for (int q = 0; q < T.n; ++q) {
        const edge::TgtTerm &t = T.t[q];
        const int li = paths[t.p][0], lf = paths[t.p][1], lo = paths[t.p][2];
        const edge::Block &b = block_of(t.eg);
        int mu, mm, lo2, mo;
        comp_lm(t.em, mu, mm);
        comp_lm(t.eo, lo2, mo);
        if (b.li != li || b.lam + mu != lf || lo2 != lo) return false;
        if (!recouple(li, b.lam, mu, lf, lo, lps, U)) return false;
        double u = 0.0;
        for (size_t r = 0; r < lps.size(); ++r)
            if (lps[r] == b.lp) u = U[r];
        tgt[q] = addition_coef(lf, b.lam) * u * coupling_entry(b.lp, mu, lo, t.eg - b.off - b.lp, mm, mo);
    }
    return true;
}

const EdgeTables &edge_tables()
{
    std::call_once(g_once_edge, [] {
        std::memset(&g_edge, 0, sizeof(g_edge));
        g_edge.ok[0] = build_edge<0>(g_edge.src[0], g_edge.tgt[0]);
        g_edge.ok[1] = build_edge<1>(g_edge.src[1], g_edge.tgt[1]);
        g_edge.ok[2] = build_edge<2>(g_edge.src[2], g_edge.tgt[2]);
        for (int l = 0; l <= edge::kMaxEdgeL; ++l) {
            for (int q = 0; q < edge::kMaxSrcTerms; ++q) g_edge.srcf[l][q] = (float)g_edge.src[l][q];
            for (int q = 0; q < edge::kMaxTgtTerms; ++q) g_edge.tgtf[l][q] = (float)g_edge.tgt[l][q];
        }
    });
    return g_edge;
}
}  // namespace

namespace edge {
const float *src_values(int lmax)
{
    if (lmax < 0 || lmax > kMaxEdgeL || !edge_tables().ok[lmax]) return nullptr;
    return edge_tables().srcf[lmax];
}
const float *tgt_values(int lmax)
{
    if (lmax < 0 || lmax > kMaxEdgeL || !edge_tables().ok[lmax]) return nullptr;
    return edge_tables().tgtf[lmax];
}
}  // namespace edge

const Tables &host_tables()
{
    std::call_once(g_once, build_tables);
    return g_tables;
}

const EaasCoef &eaas_table(int lmax)
{
    std::call_once(g_once_l, [] {
        for (int l = 0; l <= kMaxL; ++l) eaas_for_lmax(l, g_by_lmax[l]);
    });
    return g_by_lmax[lmax];
}

int device_cus()
{
    constexpr int kMaxDev = 64;
    static std::atomic<int> cached[kMaxDev];    // 0: not yet asked
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < kMaxDev) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < kMaxDev) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace e2v2

// ============================================================================
// C ABI
// ============================================================================
using namespace e2v2;

namespace {
thread_local std::string t_err;

e2v2_status fail(e2v2_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
e2v2_status fail(e2v2_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_err = buf;
    return s;
}
e2v2_status hip_fail(hipError_t e, const char *where)
{
    return fail(E2V2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Attention workspace layout.
struct AttnWs {
    size_t q, k, v, hp, dmat, pos4, hhat, msc, wpack, total;
};
AttnWs attn_ws(const e2v2_layer_desc &d, int n)
{
    const size_t N = (size_t)n, C = (size_t)d.channels, NC = (size_t)n_comp(d.lmax);
    const size_t s = d.storage == E2V2_BF16 ? 2 : 4;
    const size_t nd = (size_t)(n_dmat(d.lmax) > 0 ? n_dmat(d.lmax) : 1);
    AttnWs w{};
    size_t o = 0;
    w.q = o; o += al256(N * C * 4);
    w.k = o; o += al256(N * C * 4);
    w.v = o; o += al256(d.storage == E2V2_BF16 ? 0 : N * NC * C * 4);   // bf16: v stays in registers
    w.hp = o; o += al256(d.storage == E2V2_BF16 ? N * hp_row16((int)NC, (int)C) * 2 : N * NC * C * s);
    w.dmat = o; o += al256(N * nd * 4);
    w.pos4 = o; o += al256(N * 16);
    // fp32 storage: hhat; 16-bit storage: the message m in fp16 and its node scales
    w.hhat = o; o += al256(N * NC * C * (d.storage == E2V2_BF16 ? 2 : 4));
    w.msc = o; o += al256(d.storage == E2V2_BF16 ? N * 4 : 0);
    // bf16 weights packed into MFMA fragments: W_V[0..L], W_Q, W_K, W_O[0..L]
    w.wpack = o; o += al256(d.storage == E2V2_BF16 ? (size_t)(2 * (d.lmax + 1) + 2) * C * C * 2 : 0);
    w.total = o + 256;   // slack for re-aligning an unaligned base
    return w;
}

e2v2_status check_desc(const e2v2_layer_desc *d)
{
    if (!d) return fail(E2V2_ERR_ARG, "desc is NULL");
    if (d->lmax < 0 || d->lmax > kMaxL) return fail(E2V2_ERR_ARG, "lmax %d outside 0..3", d->lmax);
    if (d->heads <= 0 || d->channels <= 0 || d->channels % d->heads != 0)
        return fail(E2V2_ERR_ARG, "channels %d not a positive multiple of heads %d", d->channels, d->heads);
    if (d->channels / d->heads != 8)
        return fail(E2V2_ERR_UNSUPPORTED, "channels per head must be 8 (got %d)", d->channels / d->heads);
    if (d->heads != 4 && d->heads != 8 && d->heads != 16)
        return fail(E2V2_ERR_UNSUPPORTED, "heads must be 4, 8 or 16 (got %d)", d->heads);
    if (d->n_rbf < 2 || d->n_rbf > 64) return fail(E2V2_ERR_ARG, "n_rbf %d outside 2..64", d->n_rbf);
    if (!(d->cutoff > 0.f) || !std::isfinite(d->cutoff)) return fail(E2V2_ERR_ARG, "cutoff must be finite and > 0");
    if (d->storage != E2V2_FP32 && d->storage != E2V2_BF16) return fail(E2V2_ERR_ARG, "unknown storage dtype %d", d->storage);
    return E2V2_OK;
}
}  // namespace

extern "C" {

const char *e2v2_status_string(e2v2_status s)
{
    switch (s) {
    case E2V2_OK: return "ok";
    case E2V2_ERR_ARG: return "invalid argument";
    case E2V2_ERR_CAPACITY: return "insufficient neighbour capacity";
    case E2V2_ERR_UNSUPPORTED: return "unsupported shape";
    case E2V2_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *e2v2_last_error(void) { return t_err.c_str(); }

int32_t e2v2_num_paths(int32_t lmax)
{
    if (lmax < 0 || lmax > kMaxL) return -1;
    return path_count(lmax);
}

e2v2_status e2v2_path_table(int32_t lmax, int32_t *t)
{
    if (lmax < 0 || lmax > kMaxL) return fail(E2V2_ERR_ARG, "lmax %d outside 0..3", lmax);
    if (!t) return fail(E2V2_ERR_ARG, "table pointer is NULL");
    int p = 0;
    for (int lo = 0; lo <= lmax; ++lo)
        for (int li = 0; li <= lmax; ++li)
            for (int lf = 0; lf <= lmax; ++lf)
                if (is_path(li, lf, lo)) {
                    t[3 * p] = li; t[3 * p + 1] = lf; t[3 * p + 2] = lo;
                    ++p;
                }
    return E2V2_OK;
}

e2v2_status e2v2_eaas_coefficients(int32_t lmax, float *coef)
{
    if (lmax < 0 || lmax > kMaxL) return fail(E2V2_ERR_ARG, "lmax %d outside 0..3", lmax);
    if (!coef) return fail(E2V2_ERR_ARG, "coef is NULL");
    const EaasCoef &t = eaas_table(lmax);
    for (int p = 0; p < path_count(lmax); ++p)
        for (int e = 0; e < 2 * kMaxL + 1; ++e) coef[p * 7 + e] = t.c[p][e];
    return E2V2_OK;
}

e2v2_status e2v2_alignment_wigner(int32_t lmax, const double *r, double *d)
{
    if (lmax < 0 || lmax > kMaxL) return fail(E2V2_ERR_ARG, "lmax %d outside 0..3", lmax);
    if (!r || !d) return fail(E2V2_ERR_ARG, "NULL pointer");
    double D[n_dmat(kMaxL)];
    wigner_blocks<kMaxL>(r[0], r[1], r[2], host_tables().ds, D);
    for (int e = 0; e < n_dmat(lmax); ++e) d[e] = D[e];
    return E2V2_OK;
}

size_t e2v2_build_neighbors_workspace_bytes(int32_t n, int32_t max_neighbors)
{
    if (n < 0) return 0;
    return neighbors_ws_bytes(n, max_neighbors) + 256;
}

size_t e2v2_target_order_workspace_bytes(int32_t n)
{
    if (n < 0) return 0;
    return target_order_ws_bytes(n) + 256;
}

e2v2_status e2v2_target_order(const float *pos, int32_t n, int32_t *order, void *workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    if (n < 0 || n == INT32_MAX) return fail(E2V2_ERR_ARG, "n = %d out of range", n);
    if (n == 0) return E2V2_OK;
    if (!pos || !order || !workspace) return fail(E2V2_ERR_ARG, "NULL device pointer");
    if ((reinterpret_cast<uintptr_t>(pos) | reinterpret_cast<uintptr_t>(order)) & 3u)
        return fail(E2V2_ERR_ARG, "pos and order must be 4-byte aligned");
    if (workspace_bytes < e2v2_target_order_workspace_bytes(n))
        return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes,
                    e2v2_target_order_workspace_bytes(n));
    void *ws = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    const hipError_t e = launch_target_order(pos, n, ws, order, stream);
    if (e != hipSuccess) return hip_fail(e, "target order");
    return E2V2_OK;
}

e2v2_status e2v2_build_neighbors(const float *pos, int32_t n, float cutoff, int32_t K, int32_t *nbr_start,
                                 int32_t *nbr_len, int32_t *nbr_idx, int64_t capacity, int64_t *nnz_host,
                                 int32_t *order, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (n < 0 || n == INT32_MAX) return fail(E2V2_ERR_ARG, "n = %d out of range", n);
    if (!(cutoff > 0.f) || !std::isfinite(cutoff)) return fail(E2V2_ERR_ARG, "cutoff must be finite and > 0");
    if (K < 0 || K > 4096) return fail(E2V2_ERR_ARG, "max_neighbors %d outside 0..4096", K);
    if (K == 0 && !nnz_host) return fail(E2V2_ERR_ARG, "nnz_host is required for CSR output");
    if (capacity < 0) return fail(E2V2_ERR_ARG, "negative capacity");
    if (K > 0 && capacity < (int64_t)n * K)
        return fail(E2V2_ERR_ARG, "capacity %lld < n*K = %lld", (long long)capacity, (long long)n * K);
    if (K > 0 && (int64_t)n * K >= INT32_MAX) return fail(E2V2_ERR_ARG, "n*K exceeds int32 offsets");
    if (n == 0) {
        if (nnz_host) *nnz_host = 0;
        return E2V2_OK;
    }
    if (!pos || !nbr_start || !nbr_len || !nbr_idx || !workspace) return fail(E2V2_ERR_ARG, "NULL device pointer");
    if (!aligned16(pos) || !aligned16(nbr_start) || !aligned16(nbr_len) || !aligned16(nbr_idx) ||
        (order && !aligned16(order)))
        return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    if (workspace_bytes < e2v2_build_neighbors_workspace_bytes(n, K))
        return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, e2v2_build_neighbors_workspace_bytes(n, K));
    void *ws = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    hipError_t e = launch_neighbors_count(pos, n, cutoff, K, ws, workspace_bytes, nbr_len, order, stream);
    if (e != hipSuccess) return hip_fail(e, "neighbour grid");
    if (K == 0) {
        int64_t *nnz_dev = neighbors_nnz_slot(ws, n);
        e = launch_neighbors_scan(n, ws, nbr_start, nbr_len, nnz_dev, stream);
        if (e != hipSuccess) return hip_fail(e, "neighbour scan");
        int64_t nnz = 0;
        e = hipMemcpyAsync(&nnz, nnz_dev, sizeof nnz, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "reading nnz");
        *nnz_host = nnz;
        if (nnz > capacity)
            return fail(E2V2_ERR_CAPACITY, "need %lld neighbour slots, capacity %lld", (long long)nnz, (long long)capacity);
        if (nnz >= INT32_MAX) return fail(E2V2_ERR_CAPACITY, "nnz %lld exceeds int32 offsets", (long long)nnz);
    }
    e = launch_neighbors_fill(pos, n, cutoff, K, ws, nbr_start, nbr_len, nbr_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "neighbour fill");
    if (K > 0 && nnz_host) {
        // Sum of the row lengths, read back (the documented synchronising option).
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "synchronise");
        int32_t *lens = new int32_t[(size_t)n];
        e = hipMemcpy(lens, nbr_len, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost);
        int64_t s = 0;
        for (int i = 0; i < n; ++i) s += lens[i];
        delete[] lens;
        if (e != hipSuccess) return hip_fail(e, "reading nbr_len");
        *nnz_host = s;
    }
    return E2V2_OK;
}

e2v2_status e2v2_eaas_couple(const float *pos, const void *x, e2v2_dtype x_dtype, const float *path_w, int32_t n,
                             int32_t lmax, int32_t channels, void *y, e2v2_dtype y_dtype, hipStream_t stream)
{
    if (lmax < 0 || lmax > kMaxL) return fail(E2V2_ERR_ARG, "lmax %d outside 0..3", lmax);
    if (channels <= 0 || channels > 256 || channels % 8 != 0)
        return fail(E2V2_ERR_ARG, "channels %d must be a multiple of 8 in 8..256", channels);
    if ((x_dtype != E2V2_FP32 && x_dtype != E2V2_BF16) || (y_dtype != E2V2_FP32 && y_dtype != E2V2_BF16))
        return fail(E2V2_ERR_ARG, "unknown dtype");
    if (n < 0) return fail(E2V2_ERR_ARG, "n < 0");
    if (n == 0) return E2V2_OK;
    if (!pos || !x || !path_w || !y) return fail(E2V2_ERR_ARG, "NULL device pointer");
    if (!aligned16(pos) || !aligned16(x) || !aligned16(path_w) || !aligned16(y))
        return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    hipError_t e = launch_eaas(lmax, pos, x, x_dtype == E2V2_BF16, path_w, n, channels, y, y_dtype == E2V2_BF16 ? 1 : 0,
                               nullptr, nullptr, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "eaas kernel");
    return E2V2_OK;
}

size_t e2v2_attn_workspace_bytes(const e2v2_layer_desc *desc, int32_t n)
{
    if (!desc || n < 0 || desc->lmax < 0 || desc->lmax > kMaxL || desc->channels <= 0) return 0;
    return attn_ws(*desc, n).total;
}

}  // extern "C"

namespace {
// The layer forward in two parts that share the workspace: `prep` runs steps 2-3
// (weight packing, projections, source coupling; no neighbour list needed) and
// `agg` runs steps 4-6 (streaming attention, target coupling, output
// projection) on what `prep` left in the workspace.
e2v2_status attn_run(const e2v2_layer_desc *desc, const float *pos, const void *h, const e2v2_weights *w,
                     const int32_t *nbr_start, const int32_t *nbr_len, const int32_t *nbr_idx,
                     const int32_t *target_order, int32_t n, float *out, void *workspace, size_t workspace_bytes,
                     const e2v2_taps *taps, hipStream_t stream, bool prep, bool agg, uint16_t *out_bf16 = nullptr,
                     const uint16_t *packed_w = nullptr, bool frames_ready = false)
{
    e2v2_status st = check_desc(desc);
    if (st != E2V2_OK) return st;
    if (n < 0) return fail(E2V2_ERR_ARG, "n < 0");
    if (n == 0) return E2V2_OK;
    if (!w) return fail(E2V2_ERR_ARG, "weights is NULL");
    const void *dev_prep[] = {pos, h, w->w_q, w->w_k, w->w_v, w->w_o, w->w_src, workspace};
    // out_bf16 (bf16 storage only, used by the layer stack) replaces out
    const void *dev_agg[] = {w->w_o, w->w_rbf, w->w_tgt, nbr_start, nbr_len, nbr_idx,
                             out_bf16 ? (const void *)out_bf16 : (const void *)out, workspace};
    if (out_bf16 && desc->storage != E2V2_BF16) return fail(E2V2_ERR_ARG, "a bf16 output needs bf16 storage");
    for (int part = 0; part < 2; ++part) {
        if (part == 0 && !prep) continue;
        if (part == 1 && !agg) continue;
        for (const void *p : (part == 0 ? dev_prep : dev_agg)) {
            if (!p) return fail(E2V2_ERR_ARG, "NULL device pointer");
            if (!aligned16(p)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
        }
    }
    if (target_order && !aligned16(target_order)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    if (taps)
        for (const void *p : {(const void *)taps->q, (const void *)taps->k, (const void *)taps->v,
                              (const void *)taps->hprime, (const void *)taps->m, (const void *)taps->hhat})
            if (p && !aligned16(p)) return fail(E2V2_ERR_ARG, "tap pointers must be 16-byte aligned");
    const AttnWs L = attn_ws(*desc, n);
    if (workspace_bytes < L.total) return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, L.total);
    char *ws = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    const int lmax = desc->lmax, C = desc->channels, NC = n_comp(lmax);
    const bool bf = desc->storage == E2V2_BF16;
    const size_t wstride = (size_t)C * C * (bf ? 2 : 4);
    float *q = reinterpret_cast<float *>(ws + L.q);
    float *k = reinterpret_cast<float *>(ws + L.k);
    float *v = reinterpret_cast<float *>(ws + L.v);
    void *hp = ws + L.hp;
    float *dmat = reinterpret_cast<float *>(ws + L.dmat);
    float4 *pos4 = reinterpret_cast<float4 *>(ws + L.pos4);
    float *hhat = reinterpret_cast<float *>(ws + L.hhat);
    uint16_t *mh = reinterpret_cast<uint16_t *>(ws + L.hhat);    // 16-bit storage: the fp16 message
    float *msc = reinterpret_cast<float *>(ws + L.msc);

    hipEvent_t *ev = taps ? taps->events : nullptr;
    auto mark = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], stream) : hipSuccess; };
    hipError_t e = hipSuccess;
    // fp32 weights of degree l (fp32 storage)
    auto wv32 = [&](int l) { return reinterpret_cast<const float *>(reinterpret_cast<const char *>(w->w_v) + l * wstride); };
    auto wo32 = [&](int l) { return reinterpret_cast<const float *>(reinterpret_cast<const char *>(w->w_o) + l * wstride); };
    ProjJob jobs[kMaxL * kMaxL + 2 * kMaxL + 1 + 2];
    int nj = 0;
    // bf16 weights as MFMA fragments: packed here, or already packed by the caller
    // (the layer stack packs every layer's weights in one launch)
    uint16_t *wp = packed_w ? const_cast<uint16_t *>(packed_w) : reinterpret_cast<uint16_t *>(ws + L.wpack);
    const size_t wsz = (size_t)C * C;                 // elements per packed matrix
    if (prep) {
        e = mark(0);
        if (e != hipSuccess) return hip_fail(e, "recording stage event");
        // Step 2: projections (q, k from the l = 0 block; v per component with W_V[l]).
        if (bf && !packed_w) {
            const uint16_t *src[2 * kMaxL + 4];
            uint16_t *dst[2 * kMaxL + 4];
            int cnt = 0;
            for (int l = 0; l <= lmax; ++l) { src[cnt] = reinterpret_cast<const uint16_t *>(w->w_v) + l * wsz; dst[cnt] = wp + cnt * wsz; ++cnt; }
            src[cnt] = reinterpret_cast<const uint16_t *>(w->w_q); dst[cnt] = wp + cnt * wsz; ++cnt;
            src[cnt] = reinterpret_cast<const uint16_t *>(w->w_k); dst[cnt] = wp + cnt * wsz; ++cnt;
            for (int l = 0; l <= lmax; ++l) { src[cnt] = reinterpret_cast<const uint16_t *>(w->w_o) + l * wsz; dst[cnt] = wp + cnt * wsz; ++cnt; }
            e = launch_pack_weights(src, dst, cnt, C, stream);
            if (e != hipSuccess) return hip_fail(e, "weight packing kernel");
        }
        if (bf) {
            // Steps 2-3 fused: q, k, v on bf16 MFMA with the source EAAS applied to v in
            // registers (v itself is never stored unless tapped).
            QkvEaasArgs qa{};
            qa.h = reinterpret_cast<const uint16_t *>(h);
            qa.wv = reinterpret_cast<const uint4 *>(wp);
            qa.wq = reinterpret_cast<const uint4 *>(wp + (size_t)(lmax + 1) * wsz);
            qa.wk = reinterpret_cast<const uint4 *>(wp + (size_t)(lmax + 2) * wsz);
            qa.w_src = w->w_src; qa.pos = pos;
            qa.q = q; qa.k = k; qa.hp = reinterpret_cast<uint16_t *>(hp);
            qa.pos4 = pos4; qa.dmat = dmat;
            qa.k_tap = taps ? taps->k : nullptr;
            qa.v_tap = taps ? taps->v : nullptr;
            qa.hp_tap = taps ? taps->hprime : nullptr;
            qa.n = n;
            qa.frames_ready = frames_ready;
            qa.quad = hp_quad_layout(lmax, desc->heads, (int)C, n);
            e = launch_qkv_eaas(lmax, qa, C, stream);
            if (e == hipSuccess) e = mark(1);
            if (e == hipSuccess) e = mark(2);
            if (e != hipSuccess) return hip_fail(e, "projection + source EAAS kernel");
        } else {
            const float *h32 = reinterpret_cast<const float *>(h);
            for (int l = 0; l <= lmax; ++l)
                for (int m = 0; m < 2 * l + 1; ++m)
                    jobs[nj++] = ProjJob{h32, (long long)NC * C, wv32(l), v, (long long)NC * C, l * l + m};
            jobs[nj++] = ProjJob{h32, (long long)NC * C, reinterpret_cast<const float *>(w->w_q), q, (long long)C, 0};
            jobs[nj++] = ProjJob{h32, (long long)NC * C, reinterpret_cast<const float *>(w->w_k), k, (long long)C, 0};
            e = launch_proj(jobs, nj, n, C, stream);
            if (e == hipSuccess) e = mark(1);
            if (e != hipSuccess) return hip_fail(e, "projection kernel");
            // Step 3: source coupling h' (EAAS), per-node D blocks and padded positions.
            e = launch_eaas(lmax, pos, v, 0, w->w_src, n, C, hp, 0, taps ? taps->hprime : nullptr, dmat, pos4, stream);
            if (e == hipSuccess) e = mark(2);
            if (e != hipSuccess) return hip_fail(e, "source EAAS kernel");
        }
    }
    if (agg) {
        // Steps 4-5: streaming attention + target coupling (fp32 storage); for bf16
        // storage the streaming kernel stops at the normalised message m_i.
        AttnArgs a{};
        a.q = q; a.k = k; a.hp = hp; a.pos4 = pos4; a.dmat = dmat;
        a.nbr_start = nbr_start; a.nbr_len = nbr_len; a.nbr_idx = nbr_idx; a.order = target_order;
        a.w_rbf = w->w_rbf; a.w_tgt = w->w_tgt; a.hhat = hhat; a.mh = mh; a.msc = msc;
        a.m_tap = taps ? taps->m : nullptr;
        a.n = n; a.C = C; a.H = desc->heads; a.R = desc->n_rbf; a.cutoff = desc->cutoff;
        e = launch_attn(lmax, bf, a, stream);
        if (e == hipSuccess) e = mark(3);
        if (e != hipSuccess) return hip_fail(e, "attention kernel");
        // Step 6: output projection.
        if (bf) {
            // Step 5 (target coupling) + step 6 on whole nodes: the streaming kernel
            // left the normalised message m (fp16, node scales in msc) in the hhat buffer.
            EaasOutArgs oa{};
            oa.m = mh; oa.msc = msc; oa.dmat = dmat; oa.pos4 = pos4; oa.w_tgt = w->w_tgt;
            oa.wo = reinterpret_cast<const uint4 *>(wp + (size_t)(lmax + 3) * wsz);
            oa.out = out;
            oa.out_bf16 = out_bf16;
            oa.hhat_tap = taps ? taps->hhat : nullptr;
            oa.n = n;
            e = launch_eaas_outproj(lmax, oa, C, stream);
        } else {
            nj = 0;
            for (int l = 0; l <= lmax; ++l)
                for (int m = 0; m < 2 * l + 1; ++m)
                    jobs[nj++] = ProjJob{hhat, (long long)NC * C, wo32(l), out, (long long)NC * C, l * l + m};
            e = launch_proj(jobs, nj, n, C, stream);
        }
        if (e == hipSuccess) e = mark(4);
        if (e != hipSuccess) return hip_fail(e, "output projection kernel");
        if (taps) {
            const size_t N = (size_t)n;
            struct { void *dst; const void *src; size_t bytes; } cp[] = {
                {taps->q, q, N * C * 4}, {bf ? nullptr : taps->k, k, N * C * 4}, {bf ? nullptr : taps->v, v, N * NC * C * 4},
                {bf ? nullptr : taps->hhat, hhat, N * NC * C * 4}};
            for (auto &c : cp)
                if (c.dst) {
                    e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, stream);
                    if (e != hipSuccess) return hip_fail(e, "copying taps");
                }
        }
    }
    return E2V2_OK;
}
}  // namespace

extern "C" {

e2v2_status e2v2_attn_forward_taps(const e2v2_layer_desc *desc, const float *pos, const void *h,
                                   const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                                   const int32_t *nbr_idx, const int32_t *target_order, int32_t n, float *out,
                                   void *workspace, size_t workspace_bytes, const e2v2_taps *taps,
                                   hipStream_t stream)
{
    return attn_run(desc, pos, h, w, nbr_start, nbr_len, nbr_idx, target_order, n, out, workspace, workspace_bytes,
                    taps, stream, true, true);
}

e2v2_status e2v2_attn_prepare(const e2v2_layer_desc *desc, const float *pos, const void *h, const e2v2_weights *w,
                              int32_t n, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return attn_run(desc, pos, h, w, nullptr, nullptr, nullptr, nullptr, n, nullptr, workspace, workspace_bytes,
                    nullptr, stream, true, false);
}

e2v2_status e2v2_attn_aggregate(const e2v2_layer_desc *desc, const e2v2_weights *w, const int32_t *nbr_start,
                                const int32_t *nbr_len, const int32_t *nbr_idx, const int32_t *target_order,
                                int32_t n, float *out, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return attn_run(desc, nullptr, nullptr, w, nbr_start, nbr_len, nbr_idx, target_order, n, out, workspace,
                    workspace_bytes, nullptr, stream, false, true);
}

e2v2_status e2v2_attn_forward(const e2v2_layer_desc *desc, const float *pos, const void *h, const e2v2_weights *w,
                              const int32_t *nbr_start, const int32_t *nbr_len, const int32_t *nbr_idx,
                              const int32_t *target_order, int32_t n, float *out, void *workspace,
                              size_t workspace_bytes, hipStream_t stream)
{
    return e2v2_attn_forward_taps(desc, pos, h, w, nbr_start, nbr_len, nbr_idx, target_order, n, out, workspace,
                                  workspace_bytes, nullptr, stream);
}

}  // extern "C"

// ============================================================================
// The forward without a caller workspace, for callers that cannot allocate
// ============================================================================
namespace {
// The workspace of e2v2_attn_forward_noalloc: one array per device, held from
// the library's load to the end of the process.  In host code `scratch` names a
// host-side stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;      // 64 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];                // device address of `scratch`, per device

// This device's scratch address, looked up once per device with that device current.
e2v2_status scratch_address(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(E2V2_ERR_UNSUPPORTED, "device %d: the scratch array serves devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(E2V2_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return E2V2_OK;
}
}  // namespace

extern "C" {

e2v2_status e2v2_attn_forward_noalloc(const e2v2_layer_desc *desc, const float *pos, const void *h,
                                      const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                                      const int32_t *nbr_idx, const int32_t *target_order, int32_t n, float *out,
                                      hipStream_t stream)
{
    if (!desc) return fail(E2V2_ERR_ARG, "desc is NULL");
    e2v2_status st = check_desc(desc);
    if (st != E2V2_OK) return st;
    if (n < 0 || n == INT32_MAX) return fail(E2V2_ERR_ARG, "n = %d out of range", n);
    const size_t need = attn_ws(*desc, n).total;
    if (need > kScratchBytes)
        return fail(E2V2_ERR_CAPACITY, "n = %d needs %zu bytes of workspace; the allocation-free forward holds %zu "
                    "(use e2v2_attn_forward with a caller workspace)", n, need, kScratchBytes);
    if (n == 0) return E2V2_OK;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != E2V2_OK) return st;
    // Nothing in the workspace needs to start at zero: every region is written
    // before it is read within the call.
    return attn_run(desc, pos, h, w, nbr_start, nbr_len, nbr_idx, target_order, n, out, ws, kScratchBytes, nullptr,
                    stream, true, true);
}

}  // extern "C"

// ============================================================================
// The exact edge-equivalent form (fp32 storage, l_max <= 2)
// ============================================================================
namespace {
struct EdgeWs {
    size_t q, k, v, G, M, medge, pos4, origin, sval, tval, total;
};
EdgeWs edge_ws(const e2v2_layer_desc &d, int n)
{
    const size_t N = (size_t)n, C = (size_t)d.channels, NC = (size_t)n_comp(d.lmax);
    const int ngp = edge_padded_comps(d.lmax);
    const size_t NGP = ngp > 0 ? (size_t)ngp : 0;
    EdgeWs w{};
    size_t o = 0;
    w.q = o; o += al256(N * C * 4);
    w.k = o; o += al256(N * C * 4);
    w.v = o; o += al256(N * NC * C * 4);
    w.G = o; o += al256(N * NGP * C * 4);
    w.M = o; o += al256(N * NGP * C * 4);
    w.medge = o; o += al256(N * NC * C * 4);
    w.pos4 = o; o += al256(N * 16);
    w.origin = o; o += 256;
    w.sval = o; o += al256(sizeof(float) * edge::kMaxSrcTerms);
    w.tval = o; o += al256(sizeof(float) * edge::kMaxTgtTerms);
    w.total = o + 256;
    return w;
}
}  // namespace

extern "C" {

size_t e2v2_edge_workspace_bytes(const e2v2_layer_desc *desc, int32_t n)
{
    if (!desc || n < 0 || desc->lmax < 0 || desc->lmax > edge::kMaxEdgeL || desc->channels <= 0) return 0;
    return edge_ws(*desc, n).total;
}

e2v2_status e2v2_edge_forward(const e2v2_layer_desc *desc, const float *pos, const void *h, const e2v2_weights *w,
                              const int32_t *nbr_start, const int32_t *nbr_len, const int32_t *nbr_idx,
                              const int32_t *target_order, int32_t n, float *out, void *workspace,
                              size_t workspace_bytes, hipStream_t stream)
{
    e2v2_status st = check_desc(desc);
    if (st != E2V2_OK) return st;
    if (desc->storage != E2V2_FP32) return fail(E2V2_ERR_UNSUPPORTED, "the edge form needs fp32 storage");
    if (desc->lmax > edge::kMaxEdgeL) return fail(E2V2_ERR_UNSUPPORTED, "the edge form serves l_max <= 2");
    if (n < 0 || n == INT32_MAX) return fail(E2V2_ERR_ARG, "n = %d out of range", n);
    if (n == 0) return E2V2_OK;
    if (!w) return fail(E2V2_ERR_ARG, "weights is NULL");
    for (const void *p : {(const void *)pos, h, (const void *)w->w_q, (const void *)w->w_k, (const void *)w->w_v,
                          (const void *)w->w_o, (const void *)w->w_rbf, (const void *)w->w_src,
                          (const void *)nbr_start, (const void *)nbr_len, (const void *)nbr_idx, (const void *)out,
                          (const void *)workspace}) {
        if (!p) return fail(E2V2_ERR_ARG, "NULL device pointer");
        if (!aligned16(p)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    }
    if (target_order && !aligned16(target_order)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    const EdgeWs L = edge_ws(*desc, n);
    if (workspace_bytes < L.total) return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, L.total);
    const float *sv = edge::src_values(desc->lmax), *tv = edge::tgt_values(desc->lmax);
    if (!sv || !tv) return fail(E2V2_ERR_HIP, "edge-form coefficient tables failed their exactness check");
    char *ws = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    const int lmax = desc->lmax, C = desc->channels, NC = n_comp(lmax);
    const size_t wstride = (size_t)C * C * 4;
    float *q = reinterpret_cast<float *>(ws + L.q), *k = reinterpret_cast<float *>(ws + L.k);
    float *v = reinterpret_cast<float *>(ws + L.v), *medge = reinterpret_cast<float *>(ws + L.medge);
    auto wv32 = [&](int l) { return reinterpret_cast<const float *>(reinterpret_cast<const char *>(w->w_v) + l * wstride); };
    auto wo32 = [&](int l) { return reinterpret_cast<const float *>(reinterpret_cast<const char *>(w->w_o) + l * wstride); };
    const float *h32 = reinterpret_cast<const float *>(h);
    ProjJob jobs[kMaxL * kMaxL + 2 * kMaxL + 1 + 2];
    int nj = 0;
    for (int l = 0; l <= lmax; ++l)
        for (int m = 0; m < 2 * l + 1; ++m)
            jobs[nj++] = ProjJob{h32, (long long)NC * C, wv32(l), v, (long long)NC * C, l * l + m};
    jobs[nj++] = ProjJob{h32, (long long)NC * C, reinterpret_cast<const float *>(w->w_q), q, (long long)C, 0};
    jobs[nj++] = ProjJob{h32, (long long)NC * C, reinterpret_cast<const float *>(w->w_k), k, (long long)C, 0};
    hipError_t e = launch_proj(jobs, nj, n, C, stream);
    if (e != hipSuccess) return hip_fail(e, "projection kernel");
    e = hipMemcpyAsync(ws + L.sval, sv, sizeof(float) * edge::kMaxSrcTerms, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(ws + L.tval, tv, sizeof(float) * edge::kMaxTgtTerms, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "copying the edge-form tables");
    EdgeArgs a{};
    a.pos = pos; a.q = q; a.k = k; a.v = v; a.w_rbf = w->w_rbf; a.w_e = w->w_src;
    a.src_val = reinterpret_cast<const float *>(ws + L.sval);
    a.tgt_val = reinterpret_cast<const float *>(ws + L.tval);
    a.nbr_start = nbr_start; a.nbr_len = nbr_len; a.nbr_idx = nbr_idx; a.order = target_order;
    a.G = reinterpret_cast<float *>(ws + L.G); a.M = reinterpret_cast<float *>(ws + L.M); a.medge = medge;
    a.pos4 = reinterpret_cast<float4 *>(ws + L.pos4); a.origin = reinterpret_cast<float4 *>(ws + L.origin);
    a.n = n; a.C = C; a.H = desc->heads; a.R = desc->n_rbf; a.cutoff = desc->cutoff;
    e = launch_edge(lmax, a, stream);
    if (e != hipSuccess) return hip_fail(e, "edge-form kernels");
    nj = 0;
    for (int l = 0; l <= lmax; ++l)
        for (int m = 0; m < 2 * l + 1; ++m)
            jobs[nj++] = ProjJob{medge, (long long)NC * C, wo32(l), out, (long long)NC * C, l * l + m};
    e = launch_proj(jobs, nj, n, C, stream);
    if (e != hipSuccess) return hip_fail(e, "output projection kernel");
    return E2V2_OK;
}

int32_t e2v2_edge_coefficients(int32_t lmax, int32_t which, int32_t *idx, double *val, int32_t cap)
{
    if (lmax < 0 || lmax > edge::kMaxEdgeL || which < 0 || which > 2) return -1;
    const EdgeTables &t = edge_tables();
    if (!t.ok[lmax]) return -1;
    int cnt = 0;
    auto put = [&](std::initializer_list<int> ix, double v) {
        if (cnt < cap && idx) {
            int k = 0;
            for (int x : ix) idx[4 * cnt + k++] = x;
            while (k < 4) idx[4 * cnt + k++] = -1;
            if (val) val[cnt] = v;
        }
        ++cnt;
    };
    auto emit = [&](auto B, auto S, auto T) {
        if (which == 0)
            for (int q = 0; q < S.n; ++q) put({S.t[q].ei, S.t[q].el, S.t[q].eg}, t.src[lmax][q]);
        else if (which == 1)
            for (int q = 0; q < T.n; ++q) put({T.t[q].p, T.t[q].eg, T.t[q].em, T.t[q].eo}, t.tgt[lmax][q]);
        else
            for (int k = 0; k < B.n; ++k) put({B.b[k].li, B.b[k].lam, B.b[k].lp, B.b[k].off}, 0.0);
    };
    if (lmax == 0) emit(edge::blocks<0>(), edge::src_terms<0>(), edge::tgt_terms<0>());
    else if (lmax == 1) emit(edge::blocks<1>(), edge::src_terms<1>(), edge::tgt_terms<1>());
    else emit(edge::blocks<2>(), edge::src_terms<2>(), edge::tgt_terms<2>());
    return cnt;
}

}  // extern "C"

// ============================================================================
// Gradient of the layer with respect to its input features (fp32 storage)
// ============================================================================
namespace {
// The forward workspace (q, k, v, h', frames) followed by the gradient buffers.
struct BwdWs {
    size_t fwd, gbuf, dhh, dm, mbuf, mx, rz, dd, dq, dk, tab, tcnt, tstart, tcur, tlen, tidx;
    size_t xh, xq, xk, xv, xo;       // bf16 storage: h and W_Q, W_K, W_V, W_O widened to fp32
    size_t total;
};
// The gradient runs in fp32 storage; for bf16 storage its inputs are widened first.
e2v2_layer_desc fp32_desc(const e2v2_layer_desc &d)
{
    e2v2_layer_desc f = d;
    f.storage = E2V2_FP32;
    return f;
}
BwdWs bwd_ws(const e2v2_layer_desc &d, int n, long long max_entries)
{
    const size_t N = (size_t)n, C = (size_t)d.channels, NC = (size_t)n_comp(d.lmax), H = (size_t)d.heads;
    BwdWs w{};
    size_t o = 0;
    w.fwd = o; o += al256(attn_ws(fp32_desc(d), n).total);
    w.gbuf = o; o += al256(N * NC * C * 4);      // dL/dh'
    w.dhh = o; o += al256(N * NC * C * 4);       // dL/dhhat
    w.dm = o; o += al256(N * NC * C * 4);
    w.mbuf = o; o += al256(N * NC * C * 4);      // m (for the position gradient)
    w.mx = o; o += al256(N * H * 4);
    w.rz = o; o += al256(N * H * 4);
    w.dd = o; o += al256(N * H * 4);
    w.dq = o; o += al256(N * C * 4);
    w.dk = o; o += al256(N * C * 4);
    w.tab = o; o += al256(sizeof(float) * kMaxYTerms);
    w.tcnt = o; o += al256((N + 1) * 4);         // the transposed list
    w.tstart = o; o += al256((N + 1) * 4);
    w.tcur = o; o += al256((N + 1) * 4);
    w.tlen = o; o += al256(N * 4);
    w.tidx = o; o += al256((size_t)(max_entries > 0 ? max_entries : 1) * 4);
    if (d.storage == E2V2_BF16) {
        const size_t L1 = (size_t)d.lmax + 1;
        w.xh = o; o += al256(N * NC * C * 4);
        w.xq = o; o += al256(C * C * 4);
        w.xk = o; o += al256(C * C * 4);
        w.xv = o; o += al256(L1 * C * C * 4);
        w.xo = o; o += al256(L1 * C * C * 4);
    }
    w.total = o + 256;
    return w;
}
}  // namespace

extern "C" {

size_t e2v2_layer_backward_workspace_bytes(const e2v2_layer_desc *desc, int32_t n, int64_t max_entries)
{
    if (!desc || n < 0 || max_entries < 0 || desc->lmax < 0 || desc->lmax > kMaxL || desc->channels <= 0 ||
        desc->heads <= 0)
        return 0;
    return bwd_ws(*desc, n, max_entries).total;
}

// The layer gradient; pos_acc: add dL/dpos into grad_pos instead of writing it
// (the layer stack sums it over its layers).
static e2v2_status layer_bwd(const e2v2_layer_desc *desc, const float *pos, const void *hin, const e2v2_weights *win,
                             const int32_t *nbr_start, const int32_t *nbr_len, const int32_t *nbr_idx,
                             int64_t max_entries, int32_t symmetric, int32_t reuse_forward,
                             const int32_t *target_order, int32_t n, const float *grad_out, float *grad_h,
                             float *grad_pos, void *workspace, size_t workspace_bytes, hipStream_t stream,
                             bool pos_acc, const int32_t *src_start = nullptr, const int32_t *src_len = nullptr,
                             const int32_t *src_idx = nullptr)
{
    e2v2_status st = check_desc(desc);
    if (st != E2V2_OK) return st;
    const bool bf = desc->storage == E2V2_BF16;
    if (bf && reuse_forward)
        return fail(E2V2_ERR_UNSUPPORTED, "reuse_forward needs fp32 storage (a bf16 forward keeps h' in fp16)");
    if (n < 0) return fail(E2V2_ERR_ARG, "n < 0");
    if (max_entries < 0 || max_entries >= INT32_MAX) return fail(E2V2_ERR_ARG, "max_entries %lld out of range",
                                                                 (long long)max_entries);
    if (n == 0) return E2V2_OK;
    if (!win) return fail(E2V2_ERR_ARG, "weights is NULL");
    for (const void *p : {(const void *)pos, hin, (const void *)win->w_q, (const void *)win->w_k,
                          (const void *)win->w_v, (const void *)win->w_o, (const void *)win->w_rbf,
                          (const void *)win->w_src, (const void *)win->w_tgt, (const void *)nbr_start,
                          (const void *)nbr_len, (const void *)nbr_idx, (const void *)grad_out, (const void *)grad_h,
                          (const void *)workspace}) {
        if (!p) return fail(E2V2_ERR_ARG, "NULL device pointer");
        if (!aligned16(p)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    }
    if ((target_order && !aligned16(target_order)) || (grad_pos && !aligned16(grad_pos)))
        return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    const BwdWs B = bwd_ws(*desc, n, max_entries);
    if (workspace_bytes < B.total) return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, B.total);
    char *ws = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    // bf16 storage: the gradient of the same function in fp32 arithmetic, at the
    // bf16 values of h and of W_Q, W_K, W_V, W_O, widened exactly.
    const e2v2_layer_desc d32 = fp32_desc(*desc);
    e2v2_weights w32 = *win;
    const float *h = reinterpret_cast<const float *>(hin);
    if (bf) {
        const long long L1 = desc->lmax + 1, C2 = (long long)desc->channels * desc->channels;
        float *xh = reinterpret_cast<float *>(ws + B.xh), *xq = reinterpret_cast<float *>(ws + B.xq);
        float *xk = reinterpret_cast<float *>(ws + B.xk), *xv = reinterpret_cast<float *>(ws + B.xv);
        float *xo = reinterpret_cast<float *>(ws + B.xo);
        hipError_t e = launch_widen_bf16(hin, xh, (long long)n * n_comp(desc->lmax) * desc->channels, stream);
        if (e == hipSuccess) e = launch_widen_bf16(win->w_q, xq, C2, stream);
        if (e == hipSuccess) e = launch_widen_bf16(win->w_k, xk, C2, stream);
        if (e == hipSuccess) e = launch_widen_bf16(win->w_v, xv, L1 * C2, stream);
        if (e == hipSuccess) e = launch_widen_bf16(win->w_o, xo, L1 * C2, stream);
        if (e != hipSuccess) return hip_fail(e, "widening the bf16 inputs");
        h = xh;
        w32.w_q = xq; w32.w_k = xk; w32.w_v = xv; w32.w_o = xo;
    }
    desc = &d32;
    const e2v2_weights *w = &w32;
    const AttnWs F = attn_ws(*desc, n);
    // Steps 2-3 of the forward pass: q, k, v, h' and the per-node frames -- or, with
    // reuse_forward, those a forward call with the same arguments left at the
    // start of this workspace.
    if (!reuse_forward) {
        st = attn_run(desc, pos, h, w, nullptr, nullptr, nullptr, nullptr, n, nullptr, ws + B.fwd, F.total, nullptr,
                      stream, true, false);
        if (st != E2V2_OK) return st;
    }
    char *fw = ws + B.fwd;          // 256-aligned already, so attn_run used the same base
    const float *q = reinterpret_cast<const float *>(fw + F.q);
    const float *k = reinterpret_cast<const float *>(fw + F.k);
    float *v = reinterpret_cast<float *>(fw + F.v);          // reused for dL/dv
    const float *hp = reinterpret_cast<const float *>(fw + F.hp);
    const float4 *pos4 = reinterpret_cast<const float4 *>(fw + F.pos4);
    float *gbuf = reinterpret_cast<float *>(ws + B.gbuf);
    float *dhh = reinterpret_cast<float *>(ws + B.dhh);
    float *dm = reinterpret_cast<float *>(ws + B.dm);
    float *dq = reinterpret_cast<float *>(ws + B.dq);
    float *dk = reinterpret_cast<float *>(ws + B.dk);
    const int L = desc->lmax, C = desc->channels, NC = n_comp(L);
    const size_t wstride = (size_t)C * C * 4;
    auto wsel = [&](const void *base, int l) {
        return reinterpret_cast<const float *>(reinterpret_cast<const char *>(base) + l * wstride);
    };
    ProjJob jobs[kMaxL * kMaxL + 2 * kMaxL + 1];
    int nj = 0;
    // Step 6 adjoint: dL/dhhat^l = g^l W_O[l]^T.
    for (int l = 0; l <= L; ++l)
        for (int m = 0; m < 2 * l + 1; ++m)
            jobs[nj++] = ProjJob{grad_out, (long long)NC * C, wsel(w->w_o, l), dhh, (long long)NC * C, l * l + m, 1, 0};
    hipError_t e = launch_proj(jobs, nj, n, C, stream);
    if (e != hipSuccess) return hip_fail(e, "output projection adjoint");
    // Step 5 adjoint: dL/dm = EAAS^T with the target's own frame and w_tgt.
    e = launch_eaas_adjoint(L, pos, dhh, w->w_tgt, n, C, dm, stream);
    if (e != hipSuccess) return hip_fail(e, "target coupling adjoint");
    // Step 4 adjoint: dq (target pass), dL/dh' and dk (source pass, over the transposed
    // list; a symmetric list is its own transpose).
    AttnBwdArgs a{};
    if (src_start) {                 // a transposed list the caller built (the stack, once per cutoff)
        a.src_start = src_start; a.src_len = src_len; a.src_idx = src_idx;
    } else if (symmetric) {
        a.src_start = nbr_start; a.src_len = nbr_len; a.src_idx = nbr_idx;
    } else {
        int32_t *tstart = reinterpret_cast<int32_t *>(ws + B.tstart);
        int32_t *tlen = reinterpret_cast<int32_t *>(ws + B.tlen);
        int32_t *tidx = reinterpret_cast<int32_t *>(ws + B.tidx);
        e = launch_transpose_list(nbr_start, nbr_len, nbr_idx, n, max_entries,
                                  reinterpret_cast<int32_t *>(ws + B.tcnt), tstart,
                                  reinterpret_cast<int32_t *>(ws + B.tcur), tidx, tlen, stream);
        if (e != hipSuccess) return hip_fail(e, "transposed list");
        a.src_start = tstart; a.src_len = tlen; a.src_idx = tidx;
    }
    a.q = q; a.k = k; a.hp = hp; a.pos4 = pos4; a.dm = dm;
    a.nbr_start = nbr_start; a.nbr_len = nbr_len; a.nbr_idx = nbr_idx; a.order = target_order;
    a.w_rbf = w->w_rbf;
    a.mx = reinterpret_cast<float *>(ws + B.mx);
    a.rz = reinterpret_cast<float *>(ws + B.rz);
    a.dd = reinterpret_cast<float *>(ws + B.dd);
    a.dq = dq; a.dk = dk; a.dhp = gbuf;
    a.grad_pos = grad_pos;
    a.pos_acc = pos_acc;
    a.m = reinterpret_cast<float *>(ws + B.mbuf);
    a.n = n; a.C = C; a.H = desc->heads; a.R = desc->n_rbf; a.cutoff = desc->cutoff;
    e = launch_attn_bwd(L, a, stream);
    if (e != hipSuccess) return hip_fail(e, "attention adjoint");
    if (grad_pos && L > 0) {
        // The encoding terms of dL/dpos, before dL/dv overwrites v.
        float *tval = reinterpret_cast<float *>(ws + B.tab);
        e = hipMemcpyAsync(tval, ygrad_values(L), sizeof(float) * kMaxYTerms, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "copying the coupling table");
        PosGradArgs pa{};
        pa.pos = pos; pa.v = v; pa.dhp = gbuf; pa.m = a.m; pa.dhhat = dhh;
        pa.w_src = w->w_src; pa.w_tgt = w->w_tgt; pa.tval = tval; pa.grad_pos = grad_pos;
        pa.n = n; pa.C = C; pa.H = desc->heads;
        e = launch_pos_grad(L, pa, stream);
        if (e != hipSuccess) return hip_fail(e, "encoding gradient");
    }
    // Step 3 adjoint: dL/dv = EAAS^T with the source's own frame and w_src.
    e = launch_eaas_adjoint(L, pos, gbuf, w->w_src, n, C, v, stream);
    if (e != hipSuccess) return hip_fail(e, "source coupling adjoint");
    // Step 2 adjoint: dh^l = dv^l W_V[l]^T, then dh^0 += dq W_Q^T and dh^0 += dk W_K^T
    // (launches in stream order: the accumulating jobs write the rows of the first).
    nj = 0;
    for (int l = 0; l <= L; ++l)
        for (int m = 0; m < 2 * l + 1; ++m)
            jobs[nj++] = ProjJob{v, (long long)NC * C, wsel(w->w_v, l), grad_h, (long long)NC * C, l * l + m, 1, 0};
    e = launch_proj(jobs, nj, n, C, stream);
    ProjJob jq{dq, (long long)C, reinterpret_cast<const float *>(w->w_q), grad_h, (long long)NC * C, 0, 1, 1};
    ProjJob jk{dk, (long long)C, reinterpret_cast<const float *>(w->w_k), grad_h, (long long)NC * C, 0, 1, 1};
    if (e == hipSuccess) e = launch_proj(&jq, 1, n, C, stream);
    if (e == hipSuccess) e = launch_proj(&jk, 1, n, C, stream);
    if (e != hipSuccess) return hip_fail(e, "input projection adjoint");
    return E2V2_OK;
}

e2v2_status e2v2_layer_backward(const e2v2_layer_desc *desc, const float *pos, const void *h, const e2v2_weights *w,
                                const int32_t *nbr_start, const int32_t *nbr_len, const int32_t *nbr_idx,
                                int64_t max_entries, int32_t symmetric, int32_t reuse_forward,
                                const int32_t *target_order, int32_t n,
                                const float *grad_out, float *grad_h, float *grad_pos, void *workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    return layer_bwd(desc, pos, h, w, nbr_start, nbr_len, nbr_idx, max_entries, symmetric, reuse_forward,
                     target_order, n, grad_out, grad_h, grad_pos, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

// ============================================================================
// Neighbour reuse and the layer stack
// ============================================================================
namespace {
constexpr int kMaxStackLayers = 16;

// Distinct layer cutoffs, largest first.
int distinct_cutoffs(int L, const e2v2_layer_desc *d, float *cut)
{
    int nc = 0;
    for (int l = 0; l < L; ++l) {
        bool seen = false;
        for (int k = 0; k < nc; ++k) seen = seen || cut[k] == d[l].cutoff;
        if (!seen) cut[nc++] = d[l].cutoff;
    }
    std::sort(cut, cut + nc, [](float a, float b) { return a > b; });
    return nc;
}
int cutoff_index(int nc, const float *cut, float c)
{
    for (int k = 0; k < nc; ++k)
        if (cut[k] == c) return k;
    return -1;
}

// Persistent state: reference positions, target order, row starts, the
// displacement slot, then per distinct cutoff the row lengths and entries.
struct StackState {
    size_t ref, order, start, disp, lists, per_list, len_off, total;
    int ncut;
    float cut[kMaxStackLayers];
};
StackState stack_state(int L, const e2v2_layer_desc *d, int n, int K)
{
    StackState s{};
    s.ncut = distinct_cutoffs(L, d, s.cut);
    const size_t N = (size_t)n;
    size_t o = 0;
    s.ref = o; o += al256(N * 12);
    s.order = o; o += al256(N * 4);
    s.start = o; o += al256(N * 4);
    s.disp = o; o += 256;
    s.lists = o;
    s.len_off = al256(N * 4);
    s.per_list = s.len_off + al256(N * (size_t)K * 4);
    o += s.per_list * (size_t)s.ncut;
    s.total = o + 256;
    return s;
}

// Scratch: neighbour build workspace, one layer workspace (the largest) and two
// feature buffers in the storage dtype for the layers' outputs.
struct StackWs {
    size_t nbws, nbws_bytes, lws, lws_bytes, f0, f1, wpk, wpk_layer, total;
};
StackWs stack_ws(int L, const e2v2_layer_desc *d, int n, int K)
{
    StackWs w{};
    const size_t feat = (size_t)n * (size_t)n_comp(d[0].lmax) * (size_t)d[0].channels;
    size_t o = 0;
    w.nbws = o; w.nbws_bytes = e2v2_build_neighbors_workspace_bytes(n, K); o += al256(w.nbws_bytes);
    size_t lb = 0;
    for (int l = 0; l < L; ++l) lb = std::max(lb, attn_ws(d[l], n).total);
    w.lws = o; w.lws_bytes = lb; o += al256(lb);
    // the previous layer's output as the next layer's input, ping-pong: fp32 buffers
    // for fp32 storage, bf16 buffers (written by the output kernel) for bf16
    const size_t es = d[0].storage == E2V2_BF16 ? 2 : 4;
    w.f0 = o; o += al256(L > 1 ? feat * es : 0);
    w.f1 = o; o += al256(L > 2 ? feat * es : 0);
    // bf16: every layer's weights as MFMA fragments (W_V[0..L], W_Q, W_K, W_O[0..L])
    const size_t C = (size_t)d[0].channels;
    w.wpk_layer = d[0].storage == E2V2_BF16 ? al256((size_t)(2 * (d[0].lmax + 1) + 2) * C * C * 2) : 0;
    w.wpk = o; o += w.wpk_layer * (size_t)L;
    w.total = o + 256;
    return w;
}

e2v2_status check_stack(int L, const e2v2_layer_desc *descs, const e2v2_weights *weights, int n, int K)
{
    if (L < 1 || L > kMaxStackLayers) return fail(E2V2_ERR_ARG, "n_layers %d outside 1..%d", L, kMaxStackLayers);
    if (!descs) return fail(E2V2_ERR_ARG, "descs is NULL");
    for (int l = 0; l < L; ++l) {
        e2v2_status st = check_desc(&descs[l]);
        if (st != E2V2_OK) return st;
        if (descs[l].lmax != descs[0].lmax || descs[l].channels != descs[0].channels ||
            descs[l].storage != descs[0].storage)
            return fail(E2V2_ERR_ARG, "layer %d differs from layer 0 in lmax, channels or storage", l);
        if (weights && !weights[l].w_q) return fail(E2V2_ERR_ARG, "weights[%d] has NULL pointers", l);
    }
    if (n < 0 || n == INT32_MAX) return fail(E2V2_ERR_ARG, "n = %d out of range", n);
    if (K < 1 || K > 4096) return fail(E2V2_ERR_ARG, "max_neighbors %d outside 1..4096", K);
    if ((int64_t)n * K >= INT32_MAX) return fail(E2V2_ERR_ARG, "n*K exceeds int32 offsets");
    return E2V2_OK;
}
}  // namespace

namespace {
// Workspace of the stack gradient: one layer-gradient workspace (which also serves
// the forward recomputation), the fp32 inputs of layers 1..L-1, two gradient buffers.
struct StackBwdWs {
    size_t bws, bws_bytes, x, per_x, g0, g1, tl, per_tl, total;
};
StackBwdWs stack_bwd_ws(int L, const e2v2_layer_desc *d, int n, int K)
{
    StackBwdWs w{};
    size_t o = 0, mb = 0;
    for (int l = 0; l < L; ++l) mb = std::max(mb, bwd_ws(d[l], n, (long long)n * K).total);
    const size_t feat = al256((size_t)n * n_comp(d[0].lmax) * d[0].channels * 4);
    w.bws = o; w.bws_bytes = mb; o += al256(mb);
    w.x = o; w.per_x = feat; o += feat * (size_t)(L > 1 ? L - 1 : 0);
    w.g0 = o; o += feat;
    w.g1 = o; o += feat;
    // one transposed list per distinct cutoff: cnt, start, cur [n + 1], len [n], idx [n K]
    float cut[kMaxStackLayers];
    const int ncut = distinct_cutoffs(L, d, cut);
    const size_t N1 = al256(((size_t)n + 1) * 4);
    w.tl = o; w.per_tl = 3 * N1 + al256((size_t)n * 4) + al256((size_t)n * K * 4);
    o += w.per_tl * (size_t)ncut;
    w.total = o + 256;
    return w;
}

}  // namespace

extern "C" {

e2v2_status e2v2_filter_neighbors(const float *pos, int32_t n, float cutoff, const int32_t *nbr_start,
                                  const int32_t *nbr_len, const int32_t *nbr_idx, int32_t *out_len,
                                  int32_t *out_idx, hipStream_t stream)
{
    if (n < 0 || n == INT32_MAX) return fail(E2V2_ERR_ARG, "n = %d out of range", n);
    if (!(cutoff > 0.f) || !std::isfinite(cutoff)) return fail(E2V2_ERR_ARG, "cutoff must be finite and > 0");
    if (n == 0) return E2V2_OK;
    for (const void *p : {(const void *)pos, (const void *)nbr_start, (const void *)nbr_len, (const void *)nbr_idx,
                          (const void *)out_len, (const void *)out_idx}) {
        if (!p) return fail(E2V2_ERR_ARG, "NULL device pointer");
        if (!aligned16(p)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    }
    hipError_t e = launch_filter_rows(pos, n, cutoff, nbr_start, nbr_len, nbr_idx, out_len, out_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "neighbour filter kernel");
    return E2V2_OK;
}

e2v2_status e2v2_max_displacement2(const float *pos, const float *ref, int32_t n, double *max_d2, hipStream_t stream)
{
    if (n < 0) return fail(E2V2_ERR_ARG, "n < 0");
    if (!max_d2 || (n > 0 && (!pos || !ref))) return fail(E2V2_ERR_ARG, "NULL device pointer");
    if ((n > 0 && (!aligned16(pos) || !aligned16(ref))) || (reinterpret_cast<uintptr_t>(max_d2) & 7u))
        return fail(E2V2_ERR_ARG, "pos and ref must be 16-byte aligned, max_d2 8-byte aligned");
    hipError_t e = launch_max_disp2(pos, ref, n, max_d2, stream);
    if (e != hipSuccess) return hip_fail(e, "displacement kernel");
    return E2V2_OK;
}

size_t e2v2_stack_state_bytes(int32_t n_layers, const e2v2_layer_desc *descs, int32_t n, int32_t max_neighbors)
{
    if (n_layers < 1 || n_layers > kMaxStackLayers || !descs || n < 0 || max_neighbors < 1) return 0;
    return stack_state(n_layers, descs, n, max_neighbors).total;
}

size_t e2v2_stack_workspace_bytes(int32_t n_layers, const e2v2_layer_desc *descs, int32_t n, int32_t max_neighbors)
{
    if (n_layers < 1 || n_layers > kMaxStackLayers || !descs || n < 0 || max_neighbors < 1) return 0;
    for (int l = 0; l < n_layers; ++l)
        if (descs[l].lmax < 0 || descs[l].lmax > kMaxL || descs[l].channels <= 0) return 0;
    return stack_ws(n_layers, descs, n, max_neighbors).total;
}

e2v2_status e2v2_stack_forward(int32_t n_layers, const e2v2_layer_desc *descs, const e2v2_weights *weights,
                               const float *pos, const void *h, int32_t n, int32_t K, e2v2_rebuild_policy *policy,
                               void *state, size_t state_bytes, float *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    e2v2_status st = check_stack(n_layers, descs, weights, n, K);
    if (st != E2V2_OK) return st;
    if (!weights) return fail(E2V2_ERR_ARG, "weights is NULL");
    if (!policy) return fail(E2V2_ERR_ARG, "policy is NULL");
    if (policy->rebuild_every < 1) return fail(E2V2_ERR_ARG, "rebuild_every %d < 1", policy->rebuild_every);
    if (!(policy->max_displacement >= 0.f) || !std::isfinite(policy->max_displacement))
        return fail(E2V2_ERR_ARG, "max_displacement must be finite and >= 0");
    if (n == 0) return E2V2_OK;
    for (const void *p : {(const void *)pos, h, (const void *)state, (const void *)out, (const void *)workspace}) {
        if (!p) return fail(E2V2_ERR_ARG, "NULL device pointer");
        if (!aligned16(p)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    }
    const StackState S = stack_state(n_layers, descs, n, K);
    const StackWs W = stack_ws(n_layers, descs, n, K);
    if (state_bytes < S.total) return fail(E2V2_ERR_ARG, "state too small: %zu < %zu", state_bytes, S.total);
    if (workspace_bytes < W.total)
        return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, W.total);
    char *sb = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(state) + 255) & ~uintptr_t(255));
    char *wb = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    float *ref = reinterpret_cast<float *>(sb + S.ref);
    int32_t *order = reinterpret_cast<int32_t *>(sb + S.order);
    int32_t *start = reinterpret_cast<int32_t *>(sb + S.start);
    double *disp = reinterpret_cast<double *>(sb + S.disp);
    auto list_len = [&](int k) { return reinterpret_cast<int32_t *>(sb + S.lists + (size_t)k * S.per_list); };
    auto list_idx = [&](int k) { return reinterpret_cast<int32_t *>(sb + S.lists + (size_t)k * S.per_list + S.len_off); };

    // 1. rebuild decision
    bool rebuild = policy->steps_since_rebuild < 0 || policy->steps_since_rebuild >= policy->rebuild_every;
    hipError_t e = hipSuccess;
    if (!rebuild) {
        e = launch_max_disp2(pos, ref, n, disp, stream);
        double d2 = 0.0;
        if (e == hipSuccess) e = hipMemcpyAsync(&d2, disp, sizeof d2, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "displacement check");
        const double lim = (double)policy->max_displacement * (double)policy->max_displacement;
        rebuild = !(d2 <= lim);
    }
    // 2. lists at the largest cutoff, then filtered for each smaller one
    if (rebuild) {
        // with the lists, the targets' processing order until the next rebuild: a
        // Hilbert curve (paid once per rebuild, its locality used by every layer of
        // every step)
        st = e2v2_build_neighbors(pos, n, S.cut[0], K, start, list_len(0), list_idx(0), (int64_t)n * K, nullptr,
                                  order, wb + W.nbws, W.nbws_bytes, stream);
        if (st != E2V2_OK) return st;
        for (int k = 1; k < S.ncut; ++k) {
            e = launch_filter_rows(pos, n, S.cut[k], start, list_len(0), list_idx(0), list_len(k), list_idx(k), stream);
            if (e != hipSuccess) return hip_fail(e, "neighbour filter kernel");
        }
        e = hipMemcpyAsync(ref, pos, (size_t)n * 12, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "keeping the reference positions");
    }
    // 3. the layers
    // bf16 storage: the output kernel of every layer but the last writes the next
    // layer's bf16 input directly (the same rounding of the same fp32 value)
    const bool bf = descs[0].storage == E2V2_BF16;
    char *fb[2] = {wb + W.f0, wb + W.f1};
    const void *x = h;
    if (bf) {       // all layers' weights packed in one launch
        const int C = descs[0].channels, lmax = descs[0].lmax;
        const size_t wsz = (size_t)C * C;
        const uint16_t *src[kMaxStackLayers * (2 * kMaxL + 4)];
        uint16_t *dst[kMaxStackLayers * (2 * kMaxL + 4)];
        int cnt = 0;
        for (int l = 0; l < n_layers; ++l) {
            uint16_t *base = reinterpret_cast<uint16_t *>(wb + W.wpk + (size_t)l * W.wpk_layer);
            const e2v2_weights &wl = weights[l];
            if (!wl.w_v || !wl.w_q || !wl.w_k || !wl.w_o) return fail(E2V2_ERR_ARG, "NULL weight pointer in layer %d", l);
            int c = 0;
            for (int ll = 0; ll <= lmax; ++ll) { src[cnt] = reinterpret_cast<const uint16_t *>(wl.w_v) + ll * wsz; dst[cnt++] = base + (c++) * wsz; }
            src[cnt] = reinterpret_cast<const uint16_t *>(wl.w_q); dst[cnt++] = base + (c++) * wsz;
            src[cnt] = reinterpret_cast<const uint16_t *>(wl.w_k); dst[cnt++] = base + (c++) * wsz;
            for (int ll = 0; ll <= lmax; ++ll) { src[cnt] = reinterpret_cast<const uint16_t *>(wl.w_o) + ll * wsz; dst[cnt++] = base + (c++) * wsz; }
        }
        for (int b0 = 0; b0 < cnt; b0 += 64) {
            e = launch_pack_weights(src + b0, dst + b0, std::min(64, cnt - b0), C, stream);
            if (e != hipSuccess) return hip_fail(e, "weight packing kernel");
        }
    }
    for (int l = 0; l < n_layers; ++l) {
        const int k = cutoff_index(S.ncut, S.cut, descs[l].cutoff);
        const bool last = l + 1 == n_layers;
        float *y = last ? out : (bf ? nullptr : reinterpret_cast<float *>(fb[l & 1]));
        uint16_t *yb = (!last && bf) ? reinterpret_cast<uint16_t *>(fb[l & 1]) : nullptr;
        // the positions, hence the D blocks in the shared layer workspace, are those of layer 0
        const uint16_t *pk = bf ? reinterpret_cast<const uint16_t *>(wb + W.wpk + (size_t)l * W.wpk_layer) : nullptr;
        st = attn_run(&descs[l], pos, x, &weights[l], start, list_len(k), list_idx(k), order, n, y, wb + W.lws,
                      W.lws_bytes, nullptr, stream, true, true, yb, pk, l > 0);
        if (st != E2V2_OK) return st;
        x = fb[l & 1];
    }
    if (rebuild) {
        policy->steps_since_rebuild = 0;
        policy->rebuilds += 1;
    }
    policy->rebuilt = rebuild ? 1 : 0;
    if (policy->steps_since_rebuild < INT32_MAX) policy->steps_since_rebuild += 1;
    return E2V2_OK;
}

size_t e2v2_stack_backward_workspace_bytes(int32_t n_layers, const e2v2_layer_desc *descs, int32_t n,
                                           int32_t max_neighbors)
{
    if (n_layers < 1 || n_layers > kMaxStackLayers || !descs || n < 0 || max_neighbors < 1) return 0;
    for (int l = 0; l < n_layers; ++l)
        if (descs[l].lmax < 0 || descs[l].lmax > kMaxL || descs[l].channels <= 0 || descs[l].heads <= 0) return 0;
    return stack_bwd_ws(n_layers, descs, n, max_neighbors).total;
}

e2v2_status e2v2_stack_backward(int32_t n_layers, const e2v2_layer_desc *descs, const e2v2_weights *weights,
                                const float *pos, const void *h, int32_t n, int32_t K, const void *state,
                                size_t state_bytes, const e2v2_rebuild_policy *policy, const float *grad_out,
                                float *grad_h, float *grad_pos, void *workspace, size_t workspace_bytes,
                                hipStream_t stream)
{
    e2v2_status st = check_stack(n_layers, descs, weights, n, K);
    if (st != E2V2_OK) return st;
    if (!weights) return fail(E2V2_ERR_ARG, "weights is NULL");
    // the state holds lists only once a forward call has built them
    if (!policy) return fail(E2V2_ERR_ARG, "policy is NULL");
    if (policy->rebuilds < 1 || policy->steps_since_rebuild < 1)
        return fail(E2V2_ERR_ARG, "no e2v2_stack_forward call has filled the state (policy shows no rebuild)");
    if (n == 0) return E2V2_OK;
    for (const void *p : {(const void *)pos, (const void *)h, state, (const void *)grad_out, (const void *)grad_h,
                          (const void *)workspace}) {
        if (!p) return fail(E2V2_ERR_ARG, "NULL device pointer");
        if (!aligned16(p)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    }
    if (grad_pos && !aligned16(grad_pos)) return fail(E2V2_ERR_ARG, "device pointers must be 16-byte aligned");
    const StackState S = stack_state(n_layers, descs, n, K);
    const StackBwdWs W = stack_bwd_ws(n_layers, descs, n, K);
    if (state_bytes < S.total) return fail(E2V2_ERR_ARG, "state too small: %zu < %zu", state_bytes, S.total);
    if (workspace_bytes < W.total)
        return fail(E2V2_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, W.total);
    const char *sb = reinterpret_cast<const char *>((reinterpret_cast<uintptr_t>(state) + 255) & ~uintptr_t(255));
    char *wb = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    const int32_t *order = reinterpret_cast<const int32_t *>(sb + S.order);
    const int32_t *start = reinterpret_cast<const int32_t *>(sb + S.start);
    auto list_len = [&](int k) { return reinterpret_cast<const int32_t *>(sb + S.lists + (size_t)k * S.per_list); };
    auto list_idx = [&](int k) {
        return reinterpret_cast<const int32_t *>(sb + S.lists + (size_t)k * S.per_list + S.len_off);
    };
    // 1. the layers' inputs, recomputed over the lists of the last e2v2_stack_forward
    //    (in the storage dtype, as the forward passed them on: the gradient takes the
    //    bf16 rounding between layers as the identity)
    const bool bf = descs[0].storage == E2V2_BF16;
    const void *x[kMaxStackLayers];
    x[0] = h;
    for (int l = 0; l + 1 < n_layers; ++l) {
        const int k = cutoff_index(S.ncut, S.cut, descs[l].cutoff);
        char *xo = wb + W.x + (size_t)l * W.per_x;
        st = attn_run(&descs[l], pos, x[l], &weights[l], start, list_len(k), list_idx(k), order, n,
                      bf ? nullptr : reinterpret_cast<float *>(xo), wb + W.bws, W.bws_bytes, nullptr, stream, true,
                      true, bf ? reinterpret_cast<uint16_t *>(xo) : nullptr);
        if (st != E2V2_OK) return st;
        x[l + 1] = xo;
    }
    // 2. the transposed list of each distinct cutoff's list, built once
    const size_t N1 = al256(((size_t)n + 1) * 4);
    auto tl = [&](int k, int part) -> int32_t * {
        char *b = wb + W.tl + (size_t)k * W.per_tl;
        const size_t off[5] = {0, N1, 2 * N1, 3 * N1, 3 * N1 + al256((size_t)n * 4)};
        return reinterpret_cast<int32_t *>(b + off[part]);
    };
    for (int k = 0; k < S.ncut; ++k) {
        const hipError_t e = launch_transpose_list(start, list_len(k), list_idx(k), n, (long long)n * K, tl(k, 0),
                                                   tl(k, 1), tl(k, 2), tl(k, 4), tl(k, 3), stream);
        if (e != hipSuccess) return hip_fail(e, "transposed list");
    }
    // 3. the layers' gradients in reverse; dL/dpos summed over the layers
    float *gb[2] = {reinterpret_cast<float *>(wb + W.g0), reinterpret_cast<float *>(wb + W.g1)};
    const float *g = grad_out;
    for (int l = n_layers - 1; l >= 0; --l) {
        const int k = cutoff_index(S.ncut, S.cut, descs[l].cutoff);
        float *go = l == 0 ? grad_h : gb[l & 1];
        st = layer_bwd(&descs[l], pos, x[l], &weights[l], start, list_len(k), list_idx(k), (int64_t)n * K, 0, 0, order,
                       n, g, go, grad_pos, wb + W.bws, W.bws_bytes, stream, l != n_layers - 1, tl(k, 1), tl(k, 3),
                       tl(k, 4));
        if (st != E2V2_OK) return st;
        g = go;
    }
    return E2V2_OK;
}

}  // extern "C"
