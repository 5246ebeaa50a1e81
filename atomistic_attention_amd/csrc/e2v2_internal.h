// Internal definitions shared by the e2v2 kernels and the host library.
//
// Geometry conventions (E2Former-V2 explainer, section 2.1): every node carries
// an alignment rotation R with R z = r / |r|; features rotate with the real
// Wigner-D blocks D^l(R), defined by Y^l(R x) = D^l(R) Y^l(x) for the real,
// component-normalised spherical harmonics Y.  In the aligned frame the
// encoding Y^{l_f}(z) has only its m = 0 entry, sqrt(2 l_f + 1), so a tensor
// product path (l_i, l_f, l_o) becomes a one-to-one map between m values
// (section 2.2): m_i = m_o for even l_i + l_f + l_o, m_i = -m_o (with a sign
// carried by the coefficient) for odd.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace e2v2 {

constexpr int kMaxL = 3;
constexpr int kMaxPaths = 34;

__host__ __device__ constexpr int n_comp(int L) { return (L + 1) * (L + 1); }

// Floats of the concatenated D^1..D^L blocks (row-major each).
__host__ __device__ constexpr int n_dmat(int L)
{
    int s = 0;
    for (int l = 1; l <= L; ++l) s += (2 * l + 1) * (2 * l + 1);
    return s;
}
__host__ __device__ constexpr int dmat_offset(int l)
{
    int s = 0;
    for (int k = 1; k < l; ++k) s += (2 * k + 1) * (2 * k + 1);
    return s;
}

__host__ __device__ constexpr bool is_path(int li, int lf, int lo)
{
    return (li - lf <= lo) && (lf - li <= lo) && (lo <= li + lf);
}
__host__ __device__ constexpr int path_count(int L)
{
    int p = 0;
    for (int lo = 0; lo <= L; ++lo)
        for (int li = 0; li <= L; ++li)
            for (int lf = 0; lf <= L; ++lf)
                if (is_path(li, lf, lo)) ++p;
    return p;
}
// Index of (li, lf, lo) in the canonical order (l_o, then l_i, then l_f); -1 if absent.
__host__ __device__ constexpr int path_index(int L, int li, int lf, int lo)
{
    int p = 0;
    for (int a = 0; a <= L; ++a)
        for (int b = 0; b <= L; ++b)
            for (int c = 0; c <= L; ++c)
                if (is_path(b, c, a)) {
                    if (a == lo && b == li && c == lf) return p;
                    ++p;
                }
    return -1;
}

// EAAS coefficients: c[p][m_o + l_o] for the single contributing m_i.
struct EaasCoef {
    float c[kMaxPaths][2 * kMaxL + 1];
};

// Sample directions X and inverse encodings Y^l(X)^{-1} for l = 2, 3:
// D^l(R) = Y^l(R X) Y^l(X)^{-1}, exact because Y^l(R x) = D^l(R) Y^l(x).
struct DSample {
    double x2[5][3];
    double inv2[5][5];
    double x3[7][3];
    double inv3[7][7];
};

struct Tables {
    EaasCoef eaas;
    DSample ds;
};

// Built once per process (thread safe).  host_tables().eaas is indexed in the
// lmax = 3 path order; eaas_table(lmax) re-indexes it for a smaller lmax.
const Tables &host_tables();
const EaasCoef &eaas_table(int lmax);

// ----------------------------------------------------------------------------
// Real spherical harmonics of a unit vector, l = 2 and l = 3 blocks (closed forms).
__host__ __device__ inline void sh_l2(double x, double y, double z, double *o)
{
    const double s15 = 3.872983346207417, s5 = 2.23606797749979;
    o[0] = s15 * x * y;
    o[1] = s15 * y * z;
    o[2] = 0.5 * s5 * (3.0 * z * z - 1.0);
    o[3] = s15 * x * z;
    o[4] = 0.5 * s15 * (x * x - y * y);
}
__host__ __device__ inline void sh_l3(double x, double y, double z, double *o)
{
    const double a = 2.091650066335189;   // sqrt(35/8)
    const double b = 10.246950765959598;  // sqrt(105)
    const double c = 1.620185174601965;   // sqrt(21/8)
    const double d = 1.3228756555322954;  // sqrt(7)/2
    o[0] = a * y * (3.0 * x * x - y * y);
    o[1] = b * x * y * z;
    o[2] = c * y * (5.0 * z * z - 1.0);
    o[3] = d * (5.0 * z * z * z - 3.0 * z);
    o[4] = c * x * (5.0 * z * z - 1.0);
    o[5] = 0.5 * b * z * (x * x - y * y);
    o[6] = a * x * (x * x - 3.0 * y * y);
}

// Alignment rotation R = R_z(alpha) R_y(beta) taking z onto r/|r|, built from the
// direction cosines (no trigonometric calls).  Returns false for r = 0 (R = I).
__host__ __device__ inline bool alignment_rotation(double x, double y, double z, double R[3][3])
{
    double n2 = x * x + y * y + z * z;
    if (!(n2 > 0.0)) {
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b) R[a][b] = (a == b) ? 1.0 : 0.0;
        return false;
    }
    double inv = 1.0 / sqrt(n2);
    x *= inv;
    y *= inv;
    z *= inv;
    double rho = sqrt(x * x + y * y);
    double ca = 1.0, sa = 0.0;
    if (rho > 0.0) {
        ca = x / rho;
        sa = y / rho;
    }
    double cb = z, sb = rho;
    R[0][0] = ca * cb; R[0][1] = -sa; R[0][2] = ca * sb;
    R[1][0] = sa * cb; R[1][1] = ca;  R[1][2] = sa * sb;
    R[2][0] = -sb;     R[2][1] = 0.0; R[2][2] = cb;
    return true;
}

// D^1..D^L of the alignment rotation of r, fp64, row-major blocks concatenated.
template <int L, typename DS>
__host__ __device__ inline bool wigner_blocks(double x, double y, double z, const DS &ds, double *D)
{
    double R[3][3];
    bool dir = alignment_rotation(x, y, z, R);
    if (L >= 1) {
        // D^1 = P R P^T with P: (x, y, z) -> (y, z, x)
        const int s[3] = {1, 2, 0};
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b) D[a * 3 + b] = R[s[a]][s[b]];
    }
    if (L >= 2) {
        double Y[5][5];   // Y[m][s] = Y^2_m(R x_s)
        for (int sidx = 0; sidx < 5; ++sidx) {
            double px = R[0][0] * ds.x2[sidx][0] + R[0][1] * ds.x2[sidx][1] + R[0][2] * ds.x2[sidx][2];
            double py = R[1][0] * ds.x2[sidx][0] + R[1][1] * ds.x2[sidx][1] + R[1][2] * ds.x2[sidx][2];
            double pz = R[2][0] * ds.x2[sidx][0] + R[2][1] * ds.x2[sidx][1] + R[2][2] * ds.x2[sidx][2];
            double o[5];
            sh_l2(px, py, pz, o);
            for (int m = 0; m < 5; ++m) Y[m][sidx] = o[m];
        }
        double *D2 = D + dmat_offset(2);
        for (int a = 0; a < 5; ++a)
            for (int b = 0; b < 5; ++b) {
                double acc = 0.0;
                for (int sidx = 0; sidx < 5; ++sidx) acc += Y[a][sidx] * ds.inv2[sidx][b];
                D2[a * 5 + b] = acc;
            }
    }
    if (L >= 3) {
        double Y[7][7];
        for (int sidx = 0; sidx < 7; ++sidx) {
            double px = R[0][0] * ds.x3[sidx][0] + R[0][1] * ds.x3[sidx][1] + R[0][2] * ds.x3[sidx][2];
            double py = R[1][0] * ds.x3[sidx][0] + R[1][1] * ds.x3[sidx][1] + R[1][2] * ds.x3[sidx][2];
            double pz = R[2][0] * ds.x3[sidx][0] + R[2][1] * ds.x3[sidx][1] + R[2][2] * ds.x3[sidx][2];
            double o[7];
            sh_l3(px, py, pz, o);
            for (int m = 0; m < 7; ++m) Y[m][sidx] = o[m];
        }
        double *D3 = D + dmat_offset(3);
        for (int a = 0; a < 7; ++a)
            for (int b = 0; b < 7; ++b) {
                double acc = 0.0;
                for (int sidx = 0; sidx < 7; ++sidx) acc += Y[a][sidx] * ds.inv3[sidx][b];
                D3[a * 7 + b] = acc;
            }
    }
    return dir;
}

// ----------------------------------------------------------------------------
// EAAS on one channel: y = D(R) . P(D(R)^T x) with per-path weights w[p].
// D: the node's concatenated D^1..D^L (fp32).  `dir` false (r = 0) drops the
// l_f > 0 paths: the encoding of a zero vector is Y_0 = 1 only.  ADJ gives the
// adjoint map y = D . P^T (D^T x): the same rotations, each sparse coefficient
// carrying output component m_o back to input component m_i.
template <int L, bool ADJ = false>
__device__ __forceinline__ void eaas_channel(const float *__restrict__ D, const float (&x)[n_comp(L)],
                                             float (&y)[n_comp(L)], const float *w, const EaasCoef &tab,
                                             bool dir)
{
    constexpr int NC = n_comp(L);
    float xt[NC];
    xt[0] = x[0];
#pragma unroll
    for (int l = 1; l <= L; ++l) {
        const int o = l * l, k = 2 * l + 1;
        const float *Dl = D + dmat_offset(l);
#pragma unroll
        for (int b = 0; b < k; ++b) {
            float acc = 0.f;
#pragma unroll
            for (int a = 0; a < k; ++a) acc = fmaf(Dl[a * k + b], x[o + a], acc);
            xt[o + b] = acc;
        }
    }
    float loc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) loc[i] = 0.f;
    const float fdir = dir ? 1.f : 0.f;
#pragma unroll
    for (int lo = 0; lo <= L; ++lo)
#pragma unroll
        for (int li = 0; li <= L; ++li)
#pragma unroll
            for (int lf = 0; lf <= L; ++lf) {
                if (!is_path(li, lf, lo)) continue;
                const int p = path_index(L, li, lf, lo);
                const bool odd = ((li + lf + lo) & 1) != 0;
                const int mm = li < lo ? li : lo;
                const float wp = (lf > 0) ? w[p] * fdir : w[p];
#pragma unroll
                for (int mo = -mm; mo <= mm; ++mo) {
                    if (odd && mo == 0) continue;
                    const int mi = odd ? -mo : mo;
                    const int eo = lo * lo + lo + mo, ei = li * li + li + mi;
                    if constexpr (ADJ)
                        loc[ei] = fmaf(wp * tab.c[p][mo + lo], xt[eo], loc[ei]);
                    else
                        loc[eo] = fmaf(wp * tab.c[p][mo + lo], xt[ei], loc[eo]);
                }
            }
    y[0] = loc[0];
#pragma unroll
    for (int l = 1; l <= L; ++l) {
        const int o = l * l, k = 2 * l + 1;
        const float *Dl = D + dmat_offset(l);
#pragma unroll
        for (int a = 0; a < k; ++a) {
            float acc = 0.f;
#pragma unroll
            for (int b = 0; b < k; ++b) acc = fmaf(Dl[a * k + b], loc[o + b], acc);
            y[o + a] = acc;
        }
    }
}

// ----------------------------------------------------------------------------
// One multiply-add of the aligned-frame coupling: output component `out`
// receives coefficient c[p][cc] times path weight p times input component `in`;
// lf > 0 terms vanish for a node at the origin.
struct CTerm {
    int p, out, in, cc, lf;
};
template <int L>
struct CTerms {
    int n;
    CTerm t[(2 * kMaxL + 1) * kMaxPaths];
};
template <int L>
constexpr CTerms<L> couple_terms()
{
    CTerms<L> r = {};
    int n = 0;
    for (int lo = 0; lo <= L; ++lo)
        for (int li = 0; li <= L; ++li)
            for (int lf = 0; lf <= L; ++lf) {
                if (!is_path(li, lf, lo)) continue;
                const int p = path_index(L, li, lf, lo);
                const bool odd = ((li + lf + lo) & 1) != 0;
                const int mm = li < lo ? li : lo;
                for (int mo = -mm; mo <= mm; ++mo) {
                    if (odd && mo == 0) continue;
                    const int mi = odd ? -mo : mo;
                    r.t[n++] = CTerm{p, lo * lo + lo + mo, li * li + li + mi, mo + lo, lf};
                }
            }
    r.n = n;
    return r;
}

// The re-index terms' products w[p_q][c] * c[p_q][cc_q] of one channel c, in term
// order (couple_terms), staged by a workgroup of NW waves: wave w takes terms
// w, w + NW, ..., its lanes channels lane, lane + 64, ..., at dst[c * stride + q].
// w: [paths][C] fp32.  All loads are issued before the first LDS write.
template <int L>
__constant__ CTerms<L> kCoupleTerms = couple_terms<L>();
template <int L, int C, int NW>
__device__ __forceinline__ void stage_coupling(const float *__restrict__ w, const EaasCoef &tab, float *dst,
                                               int stride, int wave, int lane)
{
    constexpr int TN = couple_terms<L>().n;
    constexpr int JM = (TN + NW - 1) / NW > 0 ? (TN + NW - 1) / NW : 1;
    constexpr int PC = (C + 63) / 64;
    float x[JM][PC];
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int q = wave + NW * j;
        if (q < TN) {
            const CTerm tq = kCoupleTerms<L>.t[q];
            const float cq = tab.c[tq.p][tq.cc];
#pragma unroll
            for (int k = 0; k < PC; ++k) {
                const int c = lane + 64 * k;
                x[j][k] = c < C ? w[tq.p * C + c] * cq : 0.f;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int q = wave + NW * j;
        if (q < TN) {
#pragma unroll
            for (int k = 0; k < PC; ++k) {
                const int c = lane + 64 * k;
                if (c < C) dst[c * stride + q] = x[j][k];
            }
        }
    }
}
template <int L>
constexpr int coupling_terms() { return couple_terms<L>().n; }

// EAAS on NI channels of one node held in registers, v[e][i] (component e,
// channel i), in place: rotate into the aligned frame (D^T x), the sparse m
// re-index with the path weights, rotate back (D y).  Dn: the node's D^1..D^L
// (fp32, may live in LDS); channel i's path weights at w0 + i * wstride; fdir = 0
// drops the l_f > 0 paths (node at the origin).  Three passes over the channels
// keep one D^l block live at a time.
template <int L, int NI, typename Arr>
__device__ __forceinline__ void eaas_multi(Arr &v, const float *Dn, const float *w0, int wstride, const EaasCoef &tab,
                                           float fdir)
{
    constexpr int NC = n_comp(L), KM = 2 * L + 1;
#pragma unroll
    for (int l = 1; l <= L; ++l) {
        const int k = 2 * l + 1, o = l * l;
        float Dl[KM * KM];
#pragma unroll
        for (int r = 0; r < k * k; ++r) Dl[r] = Dn[dmat_offset(l) + r];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float tmp[KM];
#pragma unroll
            for (int b = 0; b < k; ++b) {
                float s2 = 0.f;
#pragma unroll
                for (int a = 0; a < k; ++a) s2 = fmaf(Dl[a * k + b], v[o + a][i], s2);
                tmp[b] = s2;
            }
#pragma unroll
            for (int b = 0; b < k; ++b) v[o + b][i] = tmp[b];
        }
    }
    constexpr CTerms<L> T = couple_terms<L>();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const float *w = w0 + i * wstride;
        float loc[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) loc[e] = 0.f;
#pragma unroll
        for (int q = 0; q < T.n; ++q) {
            const float wp = T.t[q].lf > 0 ? w[T.t[q].p] * fdir : w[T.t[q].p];
            loc[T.t[q].out] = fmaf(wp * tab.c[T.t[q].p][T.t[q].cc], v[T.t[q].in][i], loc[T.t[q].out]);
        }
#pragma unroll
        for (int e = 0; e < NC; ++e) v[e][i] = loc[e];
    }
#pragma unroll
    for (int l = 1; l <= L; ++l) {
        const int k = 2 * l + 1, o = l * l;
        float Dl[KM * KM];
#pragma unroll
        for (int r = 0; r < k * k; ++r) Dl[r] = Dn[dmat_offset(l) + r];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float tmp[KM];
#pragma unroll
            for (int a = 0; a < k; ++a) {
                float s2 = 0.f;
#pragma unroll
                for (int b = 0; b < k; ++b) s2 = fmaf(Dl[a * k + b], v[o + b][i], s2);
                tmp[a] = s2;
            }
#pragma unroll
            for (int a = 0; a < k; ++a) v[o + a][i] = tmp[a];
        }
    }
}

// The same with the re-index terms' products staged beforehand (stage_coupling):
// channel i's products at wc0 + i * wstride, one FMA per term; fdir = 0 drops
// the l_f > 0 paths (node at the origin): those terms are summed first and the
// partial sums scaled by fdir.
template <int L, int NI, typename Arr>
__device__ __forceinline__ void eaas_multi_pre(Arr &v, const float *Dn, const float *wc0, int wstride, float fdir)
{
    constexpr int NC = n_comp(L), KM = 2 * L + 1;
#pragma unroll
    for (int l = 1; l <= L; ++l) {
        const int k = 2 * l + 1, o = l * l;
        float Dl[KM * KM];
#pragma unroll
        for (int r = 0; r < k * k; ++r) Dl[r] = Dn[dmat_offset(l) + r];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float tmp[KM];
#pragma unroll
            for (int b = 0; b < k; ++b) {
                float s2 = 0.f;
#pragma unroll
                for (int a = 0; a < k; ++a) s2 = fmaf(Dl[a * k + b], v[o + a][i], s2);
                tmp[b] = s2;
            }
#pragma unroll
            for (int b = 0; b < k; ++b) v[o + b][i] = tmp[b];
        }
    }
    constexpr CTerms<L> T = couple_terms<L>();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const float *w = wc0 + i * wstride;
        float loc[NC];
#pragma unroll
        for (int e = 0; e < NC; ++e) loc[e] = 0.f;
#pragma unroll
        for (int q = 0; q < T.n; ++q)
            if (T.t[q].lf > 0) loc[T.t[q].out] = fmaf(w[q], v[T.t[q].in][i], loc[T.t[q].out]);
#pragma unroll
        for (int e = 0; e < NC; ++e) loc[e] *= fdir;
#pragma unroll
        for (int q = 0; q < T.n; ++q)
            if (T.t[q].lf == 0) loc[T.t[q].out] = fmaf(w[q], v[T.t[q].in][i], loc[T.t[q].out]);
#pragma unroll
        for (int e = 0; e < NC; ++e) v[e][i] = loc[e];
    }
#pragma unroll
    for (int l = 1; l <= L; ++l) {
        const int k = 2 * l + 1, o = l * l;
        float Dl[KM * KM];
#pragma unroll
        for (int r = 0; r < k * k; ++r) Dl[r] = Dn[dmat_offset(l) + r];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float tmp[KM];
#pragma unroll
            for (int a = 0; a < k; ++a) {
                float s2 = 0.f;
#pragma unroll
                for (int b = 0; b < k; ++b) s2 = fmaf(Dl[a * k + b], v[o + b][i], s2);
                tmp[a] = s2;
            }
#pragma unroll
            for (int a = 0; a < k; ++a) v[o + a][i] = tmp[a];
        }
    }
}

// ----------------------------------------------------------------------------
// Layout of 16-bit h' in the workspace: per node NC * C elements; components are
// interleaved in pairs at 4-channel granularity, so element (e, c) of a pair
// (e < 2 * (NC / 2)) sits at (e / 2) * 2C + (c / 4) * 8 + (e % 2) * 4 + c % 4, and an
// odd last component is stored plainly at (NC - 1) * C + c.
__host__ __device__ inline int hp_f16_offset(int e, int c, int NC, int C)
{
    if (e < 2 * (NC / 2)) return (e >> 1) * 2 * C + (c >> 2) * 8 + (e & 1) * 4 + (c & 3);
    return (NC - 1) * C + c;
}
// With 16-bit storage the streaming kernel reads, per node, the h' row
// (hp_row16 fp16 elements in the hp_f16_offset layout: a lane's 4 channels of a
// component pair are one 16-byte piece, of the odd last component one 8-byte
// piece) and the key row k, fp32 [C].  h' carries the node's power-of-two scale s
// (pos4[node].w): the stored fp16 values times s.
__host__ __device__ constexpr int hp_row16(int NC, int C) { return NC * C; }
// The layout read by the four-targets-per-wave kernel (attn_quad.hip), C = 128 and
// NC = 1, 4 or 9: lane a = 4 h + c (head h, c < 4) of that kernel owns, per
// component e, the dword (h'[e][8 h + c], h'[e][8 h + 4 + c]); each lane's first
// D1 = 4 floor(NC / 4) dwords lie together (lane a at 4 D1 a bytes), the
// remaining NC - D1 in a tail region after all 64 lanes' first parts.  Offset in
// fp16 elements of (e, channel ch).
__host__ __device__ inline int hp_quad_offset(int e, int ch, int NC)
{
    const int d1 = 4 * (NC / 4), d2 = NC - d1;
    const int a = 4 * (ch >> 3) + (ch & 3), f = (ch >> 2) & 1;
    return e < d1 ? a * 2 * d1 + 2 * e + f : 128 * d1 + a * 2 * d2 + 2 * (e - d1) + f;
}
// Compute units of the current device (cached per device; 256 if the query fails):
// grid caps of the kernels that loop over tiles.
int device_cus();
// Four targets per wave with the weighted sums on the matrix cores (attn_quad.hip):
// 16-bit storage, l_max <= 2, 16 heads of 8 channels, n < attn_quad_max_atoms(L).
// Whenever it applies, the projection kernel writes h' in hp_quad_offset layout.
long long attn_quad_max_atoms(int L);
inline bool hp_quad_layout(int L, int H, int C, long long n)
{
    return L <= 2 && H == 16 && C == 128 && n < attn_quad_max_atoms(L);
}


// ----------------------------------------------------------------------------
// bf16 helpers (bit patterns in uint16_t / packed in uint32_t).
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) {               // inf / nan: keep, quiet the nan
        return uint16_t((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    }
    u += 0x7fffu + ((u >> 16) & 1u);                       // round to nearest, ties to even
    return uint16_t(u >> 16);
}

// ----------------------------------------------------------------------------
// Launch helpers implemented in the .hip files (all enqueue on `stream`).
// Ascending bitonic sort of a wave's 64 E int keys held in registers: the wave's 64 E
// keys (key x = lane * E + k in register k of lane x / E) go through the
// log2(64 E) merge phases; compare-exchange partners closer than E sit in the
// same lane, farther ones in lane ^ (d / E), reached by one shuffle per key.
// FIRST > 2 starts at the phase that merges runs of FIRST / 2: the keys must then
// already form such runs, ascending where (x & FIRST / 2) == 0, else descending.
template <int E, int FIRST = 2>
__device__ __forceinline__ void wave_bitonic_sort(int (&a)[E], int lane)
{
    constexpr int N = 64 * E;
#pragma unroll
    for (int size = FIRST; size <= N; size <<= 1) {
#pragma unroll
        for (int d = size >> 1; d >= 1; d >>= 1) {
            if (d >= E) {
                const int lx = d / E;
                // size > d >= E: the direction depends on the lane only
                const bool asc = ((lane * E) & size) == 0;
                const bool keep_min = ((lane & lx) == 0) == asc;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int o = __shfl_xor(a[k], lx, 64);
                    a[k] = keep_min ? min(a[k], o) : max(a[k], o);
                }
            } else {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if (k & d) continue;
                    const bool asc = ((lane * E + k) & size) == 0;
                    const int p = a[k], q = a[k | d];
                    a[k] = asc ? min(p, q) : max(p, q);
                    a[k | d] = asc ? max(p, q) : min(p, q);
                }
            }
        }
    }
}

// Ascending sort of a bitonic sequence of 64 E keys (same register layout as
// wave_bitonic_sort): the last merge phase of the network alone.
template <int E>
__device__ __forceinline__ void wave_bitonic_merge(int (&a)[E], int lane)
{
    constexpr int N = 64 * E;
#pragma unroll
    for (int d = N >> 1; d >= 1; d >>= 1) {
        if (d >= E) {
            const int lx = d / E;
            const bool keep_min = (lane & lx) == 0;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int o = __shfl_xor(a[k], lx, 64);
                a[k] = keep_min ? min(a[k], o) : max(a[k], o);
            }
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) {
                if (k & d) continue;
                const int p = a[k], q = a[k | d];
                a[k] = min(p, q);
                a[k | d] = max(p, q);
            }
        }
    }
}

struct NbrWork;   // neighbours.hip

// y_format: 0 fp32, 1 bf16.  y_deq (optional) receives the stored values as
// fp32; dmat_out and pos4_out (optional) the node's D blocks and (x, y, z, 1).
hipError_t launch_eaas(int L, const float *pos, const void *x, int x_bf16, const float *path_w, int n, int C,
                       void *y, int y_format, float *y_deq, float *dmat_out, float4 *pos4_out, hipStream_t stream);

struct ProjJob {
    const float *a;         // A rows: a + node*a_node_stride + comp*C (elements)
    long long a_node_stride;
    const float *b;         // [C][C] weight (in, out)
    float *out;             // out + node*o_node_stride + comp*C
    long long o_node_stride;
    int comp;               // component index of the rows
    int b_trans;            // 1: multiply by b^T (the adjoint of the projection)
    int accumulate;         // 1: out += product (jobs of one launch must write disjoint rows)
};
// fp32 projections (fp32 storage).
hipError_t launch_proj(const ProjJob *jobs, int njobs, int n, int C, hipStream_t stream);
// count bf16 values (16-byte aligned) widened to fp32, exactly.
hipError_t launch_widen_bf16(const void *in, float *out, long long count, hipStream_t stream);
// bf16 weights W [C][C] (in, out) packed into v_mfma_f32_16x16x32_bf16 A fragments.
hipError_t launch_pack_weights(const uint16_t *const *w, uint16_t *const *out, int count, int C, hipStream_t stream);

// Fused q / k / v projections and source EAAS for bf16 storage: h bf16
// [n][NC][C]; wv = packed W_V[0..L] (C*C/8 uint4 each), wq, wk packed W_Q, W_K;
// w_src [P][C].  Outputs q and k [n][C] fp32; hp: h' in fp16 (hp_f16_offset
// layout, hp_row16 elements per node) with the node's scale in pos4[node].w;
// dmat [n][n_dmat(L)].
// k_tap (fp32 [n][C]), v_tap and hp_tap (fp32 [n][NC][C]) are optional: k and v
// as projected, h' as stored (dequantised).
struct QkvEaasArgs {
    const uint16_t *h;
    const uint4 *wv, *wq, *wk;
    const float *w_src, *pos;
    float *q;
    float *k;
    uint16_t *hp;
    float4 *pos4;
    float *dmat;
    float *k_tap, *v_tap, *hp_tap;
    int n;
    bool frames_ready;               // dmat already holds these positions' D blocks
    bool quad;                       // h' in hp_quad_offset layout (else hp_f16_offset)
};
hipError_t launch_qkv_eaas(int L, const QkvEaasArgs &a, int C, hipStream_t stream);

// Target coupling + output projection for bf16 storage: m fp32 [n][NC][C] (the
// normalised message), dmat [n][n_dmat(L)], pos4 [n] (x, y, z, .), w_tgt [P][C],
// wo = packed W_O[0..L]; out fp32 [n][NC][C]; hhat_tap optional fp32 [n][NC][C].
struct EaasOutArgs {
    const uint16_t *m;               // [n][NC][C] fp16 message m_i / msc[i]
    const float *msc;                // [n] power-of-two scale of m_i
    const float *dmat;
    const float4 *pos4;
    const float *w_tgt;
    const uint4 *wo;
    float *out, *hhat_tap;
    uint16_t *out_bf16;              // if set: the output in bf16 (nearest even) instead of out
    int n;
};
hipError_t launch_eaas_outproj(int L, const EaasOutArgs &a, int C, hipStream_t stream);

struct AttnArgs {
    const float *q;                  // [n][C] fp32
    const float *k;                  // [n][C] fp32
    const void *hp;                  // [n][NC][C] fp32, or fp16 (hp_row16, hp_f16_offset) scaled by pos4[j].w
    const float4 *pos4;              // [n] (x, y, z, scale of 16-bit h'_j)
    const float *dmat;               // [n][n_dmat(L)]
    const int32_t *nbr_start, *nbr_len, *nbr_idx;
    const int32_t *order;            // optional processing order of the targets
    const float *w_rbf;              // [R][H]
    const float *w_tgt;              // [P][C]
    float *hhat;                     // [n][NC][C] fp32 hhat (fp32 storage)
    uint16_t *mh;                    // [n][NC][C] fp16 message m_i / msc[i] (16-bit storage)
    float *msc;                      // [n] power-of-two scale of m_i (16-bit storage)
    float *m_tap;                    // optional [n][NC][C]
    int n, C, H, R;
    float cutoff;
};
// hp_f16s: h' is fp16 with per-node scales (else fp32).
hipError_t launch_attn(int L, int hp_f16s, const AttnArgs &a, hipStream_t stream);
// fp32 storage: one wave per target, the target coupling in the epilogue (writes hhat).
hipError_t launch_attn_f32(int L, const AttnArgs &a, hipStream_t stream);

// Adjoint of the EAAS coupling with the node's own encoding, fp32 in and out:
// y = D . P^T (D^T x) per (node, channel), frames built from pos.
hipError_t launch_eaas_adjoint(int L, const float *pos, const float *x, const float *path_w, int n, int C, float *y,
                               hipStream_t stream);

// Gradient of the streaming attention (fp32 storage).  Given dm = dL/dm (the
// gradient of the normalised message), the target pass writes, per target i and
// head, the running maximum mx of the log2-domain logits and rz = 1 / normaliser
// (mx = +inf, rz = 0 for an empty row), dd = sum_j alpha_ij dalpha_ij, and dq; the
// source pass walks row j of the transposed list (the targets i that read source
// j) and writes dhp = dL/dh' and dk.
struct AttnBwdArgs {
    const float *q, *k, *hp;         // [n][C], [n][C], [n][NC][C]
    const float4 *pos4;              // [n] (x, y, z, .)
    const float *dm;                 // [n][NC][C]
    const int32_t *nbr_start, *nbr_len, *nbr_idx;
    const int32_t *src_start, *src_len, *src_idx;  // the sources' rows: row j at src_idx[src_start[j] ..] (src_len[j])
    const int32_t *order;            // optional processing order of the nodes
    const float *w_rbf;              // [R][H]
    float *mx, *rz, *dd;             // [n][H]
    float *dq, *dk;                  // [n][C]
    float *dhp;                      // [n][NC][C]
    float *grad_pos;                 // optional [n][3]: the bias terms of dL/dpos (target pass writes, source pass adds)
    bool pos_acc;                    // the target pass adds to grad_pos instead of writing it
    float *m;                        // [n][NC][C] the message m_i, written when grad_pos is set
    int n, C, H, R;
    float cutoff;
};
hipError_t launch_attn_bwd(int L, const AttnBwdArgs &a, hipStream_t stream);

// The exact edge-equivalent form (edge.hip, edge_terms.h): fp32 storage, l_max <= 2.
// q, k [n][C] and v [n][NC][C] from the projections; G and M [n][NGP][C] (NGP =
// edge_padded_comps(L)); medge [n][NC][C] the aggregated edge products before W_O;
// pos4 [n]; origin one float4; src_val / tgt_val device copies of the host tables.
struct EdgeArgs {
    const float *pos;
    const float *q, *k, *v;
    const float *w_rbf, *w_e;
    const float *src_val, *tgt_val;
    const int32_t *nbr_start, *nbr_len, *nbr_idx, *order;
    float *G, *M, *medge;
    float4 *pos4, *origin;
    int n, C, H, R;
    float cutoff;
};
hipError_t launch_edge(int L, const EdgeArgs &a, hipStream_t stream);
int edge_padded_comps(int L);

// Entries of the real coupling tensors T_p[m_i, m_f, m_o] with l_f >= 1 that can be
// nonzero, for the encoding gradient: in the complex basis M = mu_i + mu_f, so in
// the real basis |m_o| is |m_i| + |m_f| or ||m_i| - |m_f||, and the numbers of
// sine-type (m < 0) factors among the three has the parity of l_i + l_f + l_o
// (real part for even, imaginary part for odd).  For l_max <= 2 this is exactly
// the nonzero set.  The order is fixed at compile time; the host fills the
// values in the same order.
struct YTerm {
    int p, ei, ef, eo;               // path; components l^2 + l + m of input, encoding, output
};
constexpr int kMaxYTerms = 640;
struct YTerms {
    int n;
    YTerm t[kMaxYTerms];
};
template <int L>
constexpr YTerms ygrad_terms()
{
    YTerms r = {};
    int n = 0;
    for (int lf = 1; lf <= L; ++lf)
        for (int mf = -lf; mf <= lf; ++mf)
            for (int lo = 0; lo <= L; ++lo)
                for (int li = 0; li <= L; ++li) {
                    if (!is_path(li, lf, lo)) continue;
                    const int odd = (li + lf + lo) & 1;
                    for (int mi = -li; mi <= li; ++mi)
                        for (int mo = -lo; mo <= lo; ++mo) {
                            const int ai = mi < 0 ? -mi : mi, af = mf < 0 ? -mf : mf, ao = mo < 0 ? -mo : mo;
                            const int df = ai > af ? ai - af : af - ai;
                            if (ao != ai + af && ao != df) continue;
                            if (((mi < 0) ^ (mf < 0) ^ (mo < 0)) != odd) continue;
                            r.t[n++] = YTerm{path_index(L, li, lf, lo), li * li + li + mi, lf * lf + lf + mf,
                                             lo * lo + lo + mo};
                        }
                }
    r.n = n;
    return r;
}
// Host values T_p[m_i, m_f, m_o] in the order of ygrad_terms<lmax>() (built once).
const float *ygrad_values(int lmax);

// dL/dpos += the encoding terms: dL/dY_i = sum over the source coupling (v_i, dh'_i,
// w_src) and the target coupling (m_i, dhhat_i, w_tgt) of sum_c w_p[c] T_p x[e_i][c]
// g[e_o][c], through dY(r_i / |r_i|) / dr_i.  tval: a device copy of ygrad_values(L).
struct PosGradArgs {
    const float *pos;                // [n][3]
    const float *v, *dhp, *m, *dhhat; // [n][NC][C]
    const float *w_src, *w_tgt;      // [P][C]
    const float *tval;
    float *grad_pos;                 // [n][3], accumulated into
    int n, C, H;
};
hipError_t launch_pos_grad(int L, const PosGradArgs &a, hipStream_t stream);

// Transposed list of (start, len, idx) [n rows]: tstart [n + 1], tlen [n], tidx [cap];
// cnt and cur are [n + 1] scratch.  Rows sorted by i; entries past cap are dropped.
hipError_t launch_transpose_list(const int32_t *start, const int32_t *len, const int32_t *idx, int n,
                                 long long cap, int32_t *cnt, int32_t *tstart, int32_t *cur, int32_t *tidx,
                                 int32_t *tlen, hipStream_t stream);

hipError_t launch_neighbors_count(const float *pos, int n, float cutoff, int K, void *ws, size_t ws_bytes,
                                  int32_t *nbr_len, int32_t *order_out, hipStream_t stream);
hipError_t launch_neighbors_scan(int n, void *ws, int32_t *nbr_start, int32_t *nbr_len, int64_t *nnz_dev,
                                 hipStream_t stream);
hipError_t launch_filter_rows(const float *pos, int n, float cutoff, const int32_t *start, const int32_t *len,
                              const int32_t *idx, int32_t *out_len, int32_t *out_idx, hipStream_t stream);
hipError_t launch_max_disp2(const float *pos, const float *ref, int n, double *out, hipStream_t stream);
hipError_t launch_neighbors_fill(const float *pos, int n, float cutoff, int K, void *ws, int32_t *nbr_start,
                                 int32_t *nbr_len, int32_t *nbr_idx, hipStream_t stream);
size_t neighbors_ws_bytes(int n, int K);
// Hilbert-curve order of the atoms (order.hip): workspace bytes for n atoms, and
// the launch (bounding box, indices, stable radix sort) on one stream.
size_t target_order_ws_bytes(int n);
hipError_t launch_target_order(const float *pos, int n, void *ws, int32_t *order, hipStream_t stream);
int64_t *neighbors_nnz_slot(void *ws, int n);

}  // namespace e2v2
