"""Pins of the oracle's SO(3) machinery against things other than itself:
library routines (scipy harmonics, sympy Clebsch-Gordan), closed forms,
group-theoretic invariants, and the claims the E2Former-V2 explainer makes
(section 2.2 sparsity/sign rule, section 2.3 Proposition 4.3, section 5.2
rotation determinant and CG normalisation checks)."""
import math

import numpy as np
import pytest
import scipy.special as sps

from oracle import so3

RNG = np.random.default_rng(2024)


def _rand_dirs(n):
    v = RNG.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def _rand_rot():
    a, b, g = RNG.uniform(0, 2 * math.pi), RNG.uniform(0, math.pi), RNG.uniform(0, 2 * math.pi)
    return so3.rotation_matrix(a, b, g)


def _scipy_real_sh(r, lmax):
    """Real SH from scipy's complex Condon-Shortley harmonics via the real transform."""
    u = r / np.linalg.norm(r, axis=1, keepdims=True)
    theta = np.arccos(np.clip(u[:, 2], -1, 1))
    phi = np.arctan2(u[:, 1], u[:, 0])
    cols = []
    for l in range(lmax + 1):
        Yc = np.stack([sps.sph_harm_y(l, m, theta, phi) for m in range(-l, l + 1)], axis=1)
        cols.append((so3.complex_to_real(l) @ Yc.T).T * math.sqrt(4 * math.pi))
    Y = np.concatenate(cols, axis=1)
    assert np.max(np.abs(Y.imag)) < 1e-12
    return Y.real


# ---------------------------------------------------------------- harmonics
def test_real_sh_matches_scipy():
    r = RNG.standard_normal((200, 3)) * 3.0
    ref = _scipy_real_sh(r, 4)
    assert np.max(np.abs(so3.real_sh(r, 3) - ref[:, :16])) < 1e-13
    assert np.max(np.abs(so3.real_sh_legendre(r, 4) - ref)) < 1e-12


def test_real_sh_textbook_forms():
    r = _rand_dirs(50)
    Y = so3.real_sh(r, 3)
    x, y, z = r.T
    assert np.allclose(Y[:, 0], 1.0)
    assert np.allclose(Y[:, 1:4], math.sqrt(3) * np.stack([y, z, x], 1), atol=1e-14)
    for l in range(4):
        s = np.sum(Y[:, l * l:(l + 1) ** 2] ** 2, axis=1)
        assert np.allclose(s, 2 * l + 1, atol=1e-13)
    # only m = 0 survives on the z axis (explainer section 2.1: aligned frame)
    Yz = so3.real_sh(np.array([[0.0, 0.0, 2.5]]), 3)[0]
    for l in range(4):
        blk = Yz[l * l:(l + 1) ** 2]
        assert abs(blk[l] - math.sqrt(2 * l + 1)) < 1e-14
        if l > 0:
            assert np.max(np.abs(np.delete(blk, l))) < 1e-15


def test_zero_vector_encoding():
    Y = so3.real_sh(np.zeros((1, 3)), 3)[0]
    assert Y[0] == 1.0 and np.all(Y[1:] == 0.0)


# ---------------------------------------------------------------- Clebsch-Gordan
def test_cg_matches_sympy():
    from sympy.physics.quantum.cg import CG
    worst = 0.0
    for j1 in range(4):
        for j2 in range(4):
            for J in range(abs(j1 - j2), j1 + j2 + 1):
                for m1 in range(-j1, j1 + 1):
                    for m2 in range(-j2, j2 + 1):
                        M = m1 + m2
                        if abs(M) > J:
                            continue
                        ref = float(CG(j1, m1, j2, m2, J, M).doit())
                        worst = max(worst, abs(ref - so3.cg_complex(j1, m1, j2, m2, J, M)))
    assert worst < 1e-14


def test_cg_orthonormal():
    # section 5.2 of the explainer asks to check the CG normalisation
    for j1 in range(4):
        for j2 in range(4):
            rows = []
            for J in range(abs(j1 - j2), j1 + j2 + 1):
                for M in range(-J, J + 1):
                    rows.append([so3.cg_complex(j1, m1, j2, m2, J, M)
                                 for m1 in range(-j1, j1 + 1) for m2 in range(-j2, j2 + 1)])
            A = np.array(rows)
            assert np.allclose(A @ A.T, np.eye(A.shape[0]), atol=1e-13)


# ---------------------------------------------------------------- coupling tensors
@pytest.mark.parametrize("lmax", [2, 3])
def test_coupling_equivariant(lmax):
    for _ in range(3):
        R = _rand_rot()
        for (li, lf, lo) in so3.paths(lmax):
            T = so3.coupling_tensor(li, lf, lo)
            a, b = RNG.standard_normal(2 * li + 1), RNG.standard_normal(2 * lf + 1)
            Di, Df, Do = (so3.wigner_d(R, l) for l in (li, lf, lo))
            lhs = np.einsum("ijk,i,j->k", T, Di @ a, Df @ b)
            rhs = Do @ np.einsum("ijk,i,j->k", T, a, b)
            assert np.max(np.abs(lhs - rhs)) < 1e-12, (li, lf, lo)


def test_coupling_normalised():
    for (li, lf, lo) in so3.paths(3):
        T = so3.coupling_tensor(li, lf, lo)
        assert np.allclose(np.sum(T * T, axis=(0, 1)), 1.0, atol=1e-13)


def test_coupling_closed_forms():
    a, b = RNG.standard_normal(3), RNG.standard_normal(3)   # (y, z, x) components
    T110 = so3.coupling_tensor(1, 1, 0)
    assert abs(np.einsum("ijk,i,j->k", T110, a, b)[0] + a @ b / math.sqrt(3)) < 1e-14
    T111 = so3.coupling_tensor(1, 1, 1)
    ax, bx = a[[2, 0, 1]], b[[2, 0, 1]]                       # back to (x, y, z)
    cr = np.cross(ax, bx)[[1, 2, 0]] / math.sqrt(2)           # cross product in (y, z, x)
    assert np.max(np.abs(np.einsum("ijk,i,j->k", T111, a, b) - cr)) < 1e-14
    for l in range(4):
        x = RNG.standard_normal(2 * l + 1)
        one = np.array([1.0])
        assert np.allclose(np.einsum("ijk,i,j->k", so3.coupling_tensor(0, l, l), one, x), x, atol=1e-14)
        assert np.allclose(np.einsum("ijk,i,j->k", so3.coupling_tensor(l, 0, l), x, one), x, atol=1e-14)


def test_sparsity_and_sign_rule():
    """Explainer section 2.2: with the encoding reduced to m_f = 0, output m_o takes
    only input m_i = m_o when l_i + l_f + l_o is even, and only m_i = -m_o (with a
    sign) when it is odd; no m-summation remains."""
    for (li, lf, lo) in so3.paths(3):
        E = so3.coupling_tensor(li, lf, lo)[:, lf, :]        # m_f = 0 slice
        odd = (li + lf + lo) % 2 == 1
        for i in range(2 * li + 1):
            for o in range(2 * lo + 1):
                mi, mo = i - li, o - lo
                allowed = (mi == -mo and mo != 0) if odd else (mi == mo)
                if not allowed:
                    assert abs(E[i, o]) < 1e-14, (li, lf, lo, mi, mo)
        if odd:   # antisymmetric: E(-m -> m) = -E(m -> -m)
            for m in range(1, min(li, lo) + 1):
                assert abs(E[-m + li, m + lo] + E[m + li, -m + lo]) < 1e-14


# ---------------------------------------------------------------- Wigner-D
def test_wigner_d_properties():
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)   # xyz -> yzx
    for _ in range(5):
        R1, R2 = _rand_rot(), _rand_rot()
        assert np.max(np.abs(so3.wigner_d(R1, 1) - P @ R1 @ P.T)) < 1e-13
        for l in range(4):
            D1, D2 = so3.wigner_d(R1, l), so3.wigner_d(R2, l)
            assert np.max(np.abs(D1 @ D1.T - np.eye(2 * l + 1))) < 1e-12
            # explainer section 5.2: rotation determinant ~ 1 (asks 1e-6)
            assert abs(np.linalg.det(D1) - 1.0) < 1e-12
            assert np.max(np.abs(so3.wigner_d(R1 @ R2, l) - D1 @ D2)) < 1e-12
        x = _rand_dirs(20)
        Y, YR = so3.real_sh(x, 3), so3.real_sh(x @ R1.T, 3)
        D = so3.wigner_d_blocks(R1, 3)
        assert np.max(np.abs(YR - Y @ D.T)) < 1e-12


def test_alignment_rotation():
    for r in list(RNG.standard_normal((10, 3))) + [np.array([0, 0, -2.0]), np.array([0, 0, 3.0])]:
        R = so3.alignment_rotation(r)
        assert np.allclose(R @ np.array([0, 0, 1.0]), r / np.linalg.norm(r), atol=1e-14)
        assert abs(np.linalg.det(R) - 1) < 1e-14


# ---------------------------------------------------------------- Proposition 4.3
@pytest.mark.parametrize("lmax", [0, 1, 2, 3])
def test_eaas_equals_full_cg(lmax):
    """Explainer section 2.3, Proposition 4.3: EAAS reproduces the SO(3) tensor
    product exactly (zero error up to rounding), for any roll about r."""
    C = 6
    npath = len(so3.paths(lmax))
    for trial in range(6):
        x = RNG.standard_normal(((lmax + 1) ** 2, C))
        w = RNG.standard_normal((npath, C))
        r = RNG.standard_normal(3) * RNG.uniform(0.1, 20)
        if trial == 4:
            r = np.array([0.0, 0.0, -1.7])      # beta = pi
        if trial == 5:
            r = np.zeros(3)                     # no direction
        full = so3.tensor_product(x[None], r[None], w, lmax)[0]
        for g in (0.0, 1.1):
            e = so3.eaas_couple(x, r, w, lmax, gamma=g)
            assert np.max(np.abs(e - full)) < 1e-12


# ---------------------------------------------------------------- literal path order and EAAS table
# Every (l_i, l_f, l_o) with the triangle rule, odd l_i + l_f + l_o included
# (the odd rule of the explainer's section 2.2 needs them), ordered by l_o, then
# l_i, then l_f.  Written out by hand from that rule.
PATHS_L2 = [(0, 0, 0), (1, 1, 0), (2, 2, 0),
            (0, 1, 1), (1, 0, 1), (1, 1, 1), (1, 2, 1), (2, 1, 1), (2, 2, 1),
            (0, 2, 2), (1, 1, 2), (1, 2, 2), (2, 0, 2), (2, 1, 2), (2, 2, 2)]
PATHS_L3 = [(0, 0, 0), (1, 1, 0), (2, 2, 0), (3, 3, 0),
            (0, 1, 1), (1, 0, 1), (1, 1, 1), (1, 2, 1), (2, 1, 1), (2, 2, 1), (2, 3, 1), (3, 2, 1), (3, 3, 1),
            (0, 2, 2), (1, 1, 2), (1, 2, 2), (1, 3, 2), (2, 0, 2), (2, 1, 2), (2, 2, 2), (2, 3, 2),
            (3, 1, 2), (3, 2, 2), (3, 3, 2),
            (0, 3, 3), (1, 2, 3), (1, 3, 3), (2, 1, 3), (2, 2, 3), (2, 3, 3), (3, 0, 3), (3, 1, 3), (3, 2, 3),
            (3, 3, 3)]


def test_path_order_literal():
    assert len(PATHS_L2) == 15 and len(PATHS_L3) == 34
    assert [tuple(p) for p in so3.paths(2)] == PATHS_L2
    assert [tuple(p) for p in so3.paths(3)] == PATHS_L3
    assert [tuple(p) for p in so3.paths(1)] == [(0, 0, 0), (1, 1, 0), (0, 1, 1), (1, 0, 1), (1, 1, 1)]
    assert [tuple(p) for p in so3.paths(0)] == [(0, 0, 0)]


def _eaas_table_l2():
    """The EAAS coefficients E_p(m_i -> m_o) = sqrt(2 l_f + 1) T_p[m_i, 0, m_o] at
    l_max = 2, as closed forms: the sparse re-index of the explainer's section 2.2
    (m_i = m_o for even l_i + l_f + l_o; m_i = -m_o with a sign for odd), with the
    values of the real Condon-Shortley convention (readings R4, R8), derived by
    hand from the complex Clebsch-Gordan coefficients in the real basis.  37 entries."""
    r = math.sqrt
    t = {
        (0, 0, 0): {(0, 0): 1.0},
        (0, 1, 1): {(0, 0): r(3)},
        (0, 2, 2): {(0, 0): r(5)},
        (1, 0, 1): {(m, m): 1.0 for m in (-1, 0, 1)},
        (1, 1, 0): {(0, 0): -1.0},
        (1, 1, 1): {(-1, 1): r(1.5), (1, -1): -r(1.5)},
        (1, 1, 2): {(-1, -1): r(1.5), (1, 1): r(1.5), (0, 0): r(2)},
        (1, 2, 1): {(-1, -1): r(0.5), (1, 1): r(0.5), (0, 0): -r(2)},
        (1, 2, 2): {(-1, 1): r(2.5), (1, -1): -r(2.5)},
        (2, 0, 2): {(m, m): 1.0 for m in (-2, -1, 0, 1, 2)},
        (2, 1, 1): {(-1, -1): -r(0.9), (1, 1): -r(0.9), (0, 0): -r(1.2)},
        (2, 1, 2): {(-2, 2): r(2), (-1, 1): r(0.5), (1, -1): -r(0.5), (2, -2): -r(2)},
        (2, 2, 0): {(0, 0): 1.0},
        (2, 2, 1): {(-1, 1): -r(1.5), (1, -1): r(1.5)},
        (2, 2, 2): {(-2, -2): r(10 / 7), (2, 2): r(10 / 7), (-1, -1): -r(5 / 14), (1, 1): -r(5 / 14),
                    (0, 0): -r(10 / 7)},
    }
    assert sum(len(v) for v in t.values()) == 37
    return t


def test_eaas_table_closed_forms():
    """Every entry of the m_f = 0 slice, odd paths included, equals the table; all
    other entries are zero."""
    table = _eaas_table_l2()
    assert set(table) == set(PATHS_L2)
    for (li, lf, lo), ent in table.items():
        E = math.sqrt(2 * lf + 1) * so3.coupling_tensor(li, lf, lo)[:, lf, :]
        want = np.zeros_like(E)
        for (mi, mo), v in ent.items():
            want[mi + li, mo + lo] = v
        assert np.max(np.abs(E - want)) < 1e-14, (li, lf, lo)
