"""fp64 SO(3) machinery for the oracle: real spherical harmonics, Clebsch-Gordan
coefficients, real coupling tensors and Wigner-D matrices.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module;
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.

Everything here is written from the textbook definitions, in fp64, with no
blocking or fusion:

* Real spherical harmonics of a unit direction (the "geometric encoding"
  R^(l_f)(r) of the E2Former-V2 explainer, section 2.3, Proposition 4.3):
  real combinations of the complex Condon-Shortley harmonics, scaled by
  sqrt(4 pi) so that sum_m Y_lm^2 = 2l + 1 ("component" normalisation) and
  Y_0 = 1.  Order m = -l..l.  Two independent constructions are provided --
  closed-form polynomials and associated-Legendre recurrences -- and the tests
  pin both against scipy's complex harmonics.
* Complex Clebsch-Gordan coefficients by Racah's closed formula
  (the "CG coefficients" whose normalisation the explainer's section 5.2 asks
  to check); pinned against sympy in the tests.
* The real coupling tensor T_p[m_i, m_f, m_o] of path p = (l_i, l_f, l_o):
  the complex CG tensor conjugated into the real basis, real part when
  l_i + l_f + l_o is even, imaginary part when it is odd.
* Wigner-D matrices D^l(R) defined by Y^l(R x) = D^l(R) Y^l(x), obtained by
  least squares over sample directions (exact up to rounding, because the
  relation is linear).
* ``eaas_couple``: the explainer's section 2.1 procedure (rotate the features
  into the frame whose z axis is the position vector, keep the m_f = 0 part of
  the encoding, re-index, rotate back).  The oracle's layer never calls it; it
  exists so the tests can check Proposition 4.3 (EAAS equals the full tensor
  product) against the full Clebsch-Gordan sum.
"""
from __future__ import annotations

import functools
import math
from fractions import Fraction

import numpy as np

__all__ = [
    "real_sh", "real_sh_legendre", "cg_complex", "complex_to_real", "coupling_tensor",
    "paths", "rotation_matrix", "wigner_d", "alignment_rotation", "tensor_product",
    "eaas_couple", "block_slices",
]


def block_slices(lmax: int):
    """Component index of (l, m) is l*l + l + m; block l spans [l*l, (l+1)^2)."""
    return [slice(l * l, (l + 1) * (l + 1)) for l in range(lmax + 1)]


# --------------------------------------------------------------------------
# Real spherical harmonics
# --------------------------------------------------------------------------
def _unit(r: np.ndarray):
    r = np.asarray(r, dtype=np.float64)
    nrm = np.sqrt(np.sum(r * r, axis=-1))
    safe = np.where(nrm > 0.0, nrm, 1.0)
    return r / safe[..., None], nrm


def real_sh(r: np.ndarray, lmax: int) -> np.ndarray:
    """Closed-form real SH of the direction of r, shape [..., (lmax+1)^2].

    A zero vector has no direction: it maps to Y_0 = 1 and Y_{l>0} = 0, which is
    rotation invariant and therefore keeps the layer equivariant.
    """
    u, nrm = _unit(r)
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    out = [np.ones_like(x)]
    if lmax >= 1:
        s3 = math.sqrt(3.0)
        out += [s3 * y, s3 * z, s3 * x]
    if lmax >= 2:
        s15, s5 = math.sqrt(15.0), math.sqrt(5.0)
        out += [s15 * x * y, s15 * y * z, 0.5 * s5 * (3.0 * z * z - 1.0),
                s15 * x * z, 0.5 * s15 * (x * x - y * y)]
    if lmax >= 3:
        a, b, c = math.sqrt(35.0 / 8.0), math.sqrt(105.0), math.sqrt(21.0 / 8.0)
        out += [a * y * (3 * x * x - y * y), b * x * y * z, c * y * (5 * z * z - 1),
                0.5 * math.sqrt(7.0) * (5 * z ** 3 - 3 * z), c * x * (5 * z * z - 1),
                0.5 * b * z * (x * x - y * y), a * x * (x * x - 3 * y * y)]
    if lmax >= 4:
        raise ValueError("closed forms are written for l <= 3; use real_sh_legendre")
    Y = np.stack(out, axis=-1)
    zero = nrm == 0.0
    if np.any(zero):
        Y[zero, 1:] = 0.0
    return Y


def _assoc_legendre(lmax: int, t: np.ndarray):
    """P_l^m(t) for m >= 0 including the Condon-Shortley phase (-1)^m."""
    s = np.sqrt(np.maximum(0.0, 1.0 - t * t))
    P = {}
    P[(0, 0)] = np.ones_like(t)
    for m in range(1, lmax + 1):
        P[(m, m)] = -(2 * m - 1) * s * P[(m - 1, m - 1)]
    for m in range(0, lmax):
        P[(m + 1, m)] = (2 * m + 1) * t * P[(m, m)]
    for m in range(0, lmax + 1):
        for l in range(m + 2, lmax + 1):
            P[(l, m)] = ((2 * l - 1) * t * P[(l - 1, m)] - (l + m - 1) * P[(l - 2, m)]) / (l - m)
    return P


def real_sh_legendre(r: np.ndarray, lmax: int) -> np.ndarray:
    """Real SH built from associated Legendre functions (any lmax).

    Complex Y_l^m = N_lm P_l^m(cos th) e^{i m phi} with N_lm =
    sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!).  Real: m>0 -> sqrt2 (-1)^m Re Y_l^m,
    m<0 -> sqrt2 (-1)^m Im Y_l^|m|, m=0 -> Y_l^0; all times sqrt(4 pi).
    """
    u, nrm = _unit(r)
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    phi = np.arctan2(y, x)
    P = _assoc_legendre(lmax, np.clip(z, -1.0, 1.0))
    out = []
    for l in range(lmax + 1):
        for m in range(-l, l + 1):
            am = abs(m)
            n = math.sqrt((2 * l + 1) * math.factorial(l - am) / math.factorial(l + am))
            base = n * P[(l, am)]
            if m == 0:
                out.append(base)
            elif m > 0:
                out.append(math.sqrt(2.0) * (-1) ** m * base * np.cos(am * phi))
            else:
                out.append(math.sqrt(2.0) * (-1) ** m * base * np.sin(am * phi))
    Y = np.stack(out, axis=-1)
    zero = nrm == 0.0
    if np.any(zero):
        Y[zero, 1:] = 0.0
    return Y


def complex_to_real(l: int) -> np.ndarray:
    """U with Y_real = U @ Y_complex, rows m = -l..l, columns mu = -l..l."""
    U = np.zeros((2 * l + 1, 2 * l + 1), dtype=np.complex128)
    r2 = 1.0 / math.sqrt(2.0)
    for m in range(-l, l + 1):
        i = m + l
        if m == 0:
            U[i, l] = 1.0
        elif m > 0:
            U[i, -m + l] = r2
            U[i, m + l] = (-1) ** m * r2
        else:
            U[i, m + l] = 1j * r2
            U[i, -m + l] = -1j * (-1) ** m * r2
    return U


# --------------------------------------------------------------------------
# Clebsch-Gordan coefficients (Racah's formula) and real coupling tensors
# --------------------------------------------------------------------------
@functools.lru_cache(maxsize=None)
def cg_complex(j1: int, m1: int, j2: int, m2: int, J: int, M: int) -> float:
    """<j1 m1; j2 m2 | J M> for integer angular momenta, exact rational arithmetic."""
    if m1 + m2 != M or abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    if J < abs(j1 - j2) or J > j1 + j2:
        return 0.0
    f = math.factorial
    pref = Fraction((2 * J + 1) * f(J + j1 - j2) * f(J - j1 + j2) * f(j1 + j2 - J), f(j1 + j2 + J + 1))
    pref *= f(J + M) * f(J - M) * f(j1 - m1) * f(j1 + m1) * f(j2 - m2) * f(j2 + m2)
    total = Fraction(0)
    for k in range(0, j1 + j2 + J + 1):
        args = [k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k]
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= f(a)
        total += Fraction((-1) ** k, den)
    return float(total) * math.sqrt(float(pref))


def paths(lmax: int):
    """All (l_i, l_f, l_o) with l <= lmax satisfying the triangle rule, in the
    order l_o, then l_i, then l_f (odd l_i + l_f + l_o kept: the explainer's
    section 2.2 rule for odd L_sigma needs them)."""
    return [(li, lf, lo) for lo in range(lmax + 1) for li in range(lmax + 1)
            for lf in range(lmax + 1) if abs(li - lf) <= lo <= li + lf]


@functools.lru_cache(maxsize=None)
def coupling_tensor(li: int, lf: int, lo: int) -> np.ndarray:
    """Real coupling tensor T[m_i, m_f, m_o] of the SO(3) tensor product.

    T = sum conj(U_li) conj(U_lf) U_lo C(l_i mu_i; l_f mu_f | l_o mu_o);
    real part for even l_i + l_f + l_o, imaginary part for odd.
    (x (x) y)_{m_o} = sum_{m_i, m_f} T[m_i, m_f, m_o] x_{m_i} y_{m_f}.
    """
    C = np.zeros((2 * li + 1, 2 * lf + 1, 2 * lo + 1))
    for a in range(-li, li + 1):
        for b in range(-lf, lf + 1):
            M = a + b
            if abs(M) <= lo:
                C[a + li, b + lf, M + lo] = cg_complex(li, a, lf, b, lo, M)
    Ui, Uf, Uo = complex_to_real(li), complex_to_real(lf), complex_to_real(lo)
    T = np.einsum("ia,jb,kc,abc->ijk", Ui.conj(), Uf.conj(), Uo, C)
    if (li + lf + lo) % 2 == 0:
        assert np.max(np.abs(T.imag)) < 1e-12
        T = T.real
    else:
        assert np.max(np.abs(T.real)) < 1e-12
        T = T.imag
    T = np.ascontiguousarray(T)
    T.setflags(write=False)
    return T


def tensor_product(x: np.ndarray, r: np.ndarray, w: np.ndarray, lmax: int) -> np.ndarray:
    """Full (dense Clebsch-Gordan) depthwise tensor product with the encoding of r.

    out^{l_o}[n, m_o, c] = sum_p w[p, c] sum_{m_i, m_f} T_p[m_i, m_f, m_o]
                           x^{l_i}[n, m_i, c] Y^{l_f}_{m_f}(r_n)
    x: [n, (L+1)^2, C]; r: [n, 3]; w: [n_paths, C].  No EAAS.
    """
    x = np.asarray(x, dtype=np.float64)
    Y = real_sh(r, lmax)
    sl = block_slices(lmax)
    out = np.zeros_like(x)
    for p, (li, lf, lo) in enumerate(paths(lmax)):
        T = coupling_tensor(li, lf, lo)
        term = np.einsum("ijk,nic,nj->nkc", T, x[:, sl[li], :], Y[:, sl[lf]], optimize=True)
        out[:, sl[lo], :] += term * w[p][None, None, :]
    return out


# --------------------------------------------------------------------------
# Rotations and Wigner-D
# --------------------------------------------------------------------------
def rotation_matrix(alpha: float, beta: float, gamma: float = 0.0) -> np.ndarray:
    """R = R_z(alpha) R_y(beta) R_z(gamma)."""
    def rz(a):
        c, s = math.cos(a), math.sin(a)
        return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])

    def ry(b):
        c, s = math.cos(b), math.sin(b)
        return np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]])
    return rz(alpha) @ ry(beta) @ rz(gamma)


def alignment_rotation(r: np.ndarray, gamma: float = 0.0) -> np.ndarray:
    """A rotation taking the z axis onto the direction of r (explainer, section 2.1)."""
    r = np.asarray(r, dtype=np.float64)
    alpha = math.atan2(r[1], r[0])
    beta = math.atan2(math.hypot(r[0], r[1]), r[2])
    return rotation_matrix(alpha, beta, gamma)


_SAMPLE_DIRS = np.random.default_rng(12345).standard_normal((64, 3))


def wigner_d(R: np.ndarray, l: int) -> np.ndarray:
    """D^l(R) with Y^l(R x) = D^l(R) Y^l(x) for every direction x (least squares)."""
    X = _SAMPLE_DIRS
    sl = block_slices(l)[l]
    A = real_sh_legendre(X, l)[:, sl]          # [S, 2l+1]
    B = real_sh_legendre(X @ np.asarray(R).T, l)[:, sl]
    # B = A D^T  ->  D^T = lstsq(A, B)
    Dt, *_ = np.linalg.lstsq(A, B, rcond=None)
    return Dt.T


def wigner_d_blocks(R: np.ndarray, lmax: int) -> np.ndarray:
    """Block-diagonal D(R) over all components, [(L+1)^2, (L+1)^2]."""
    n = (lmax + 1) ** 2
    D = np.zeros((n, n))
    for l, sl in enumerate(block_slices(lmax)):
        D[sl, sl] = wigner_d(R, l)
    return D


# --------------------------------------------------------------------------
# EAAS as the explainer's section 2.1 describes it (used only to test Prop 4.3)
# --------------------------------------------------------------------------
def eaas_couple(x: np.ndarray, r: np.ndarray, w: np.ndarray, lmax: int, gamma: float = 0.0) -> np.ndarray:
    """Tensor product of one node's features with the encoding of r, via EAAS.

    1. R: a rotation taking z onto r (any roll gamma about r gives the same result);
    2. x~ = D(R)^T x  (features in the aligned frame);
    3. in that frame Y^{l_f}(z) has only its m_f = 0 entry, sqrt(2 l_f + 1), so the
       product keeps the single slice T_p[:, m_f=0, :] -- an m re-indexing;
    4. rotate back with D(R).
    x: [(L+1)^2, C]; r: [3]; w: [n_paths, C].
    """
    x = np.asarray(x, dtype=np.float64)
    sl = block_slices(lmax)
    zero = not np.any(np.asarray(r) != 0.0)
    R = np.eye(3) if zero else alignment_rotation(r, gamma)
    D = wigner_d_blocks(R, lmax)
    xt = D.T @ x
    local = np.zeros_like(x)
    for p, (li, lf, lo) in enumerate(paths(lmax)):
        if zero and lf > 0:
            continue
        E = math.sqrt(2 * lf + 1) * coupling_tensor(li, lf, lo)[:, lf, :]   # [m_i, m_o]
        local[sl[lo]] += (E.T @ xt[sl[li]]) * w[p][None, :]
    return D @ local
