"""Pins of the edge-form oracle (oracle/edge.py) against things other than itself:
polynomial closed forms of the solid harmonics, invariance under a common
translation (the edge form sees only r_j - r_i), rotation equivariance, and the
l <= 1 paths written out by hand with dot and cross products."""
import math

import numpy as np
import pytest

from oracle import edge, layer, so3

RNG = np.random.default_rng(606)


def _weights(n, C, H, R, L, seed, side=6.0):
    rng = np.random.default_rng(seed)
    P = len(so3.paths(L))
    nc = (L + 1) ** 2
    return dict(pos=rng.uniform(-side / 2, side / 2, (n, 3)).astype(np.float32).astype(np.float64),
                h=rng.standard_normal((n, nc, C)),
                w_q=rng.standard_normal((C, C)) / math.sqrt(C), w_k=rng.standard_normal((C, C)) / math.sqrt(C),
                w_v=rng.standard_normal((L + 1, C, C)) / math.sqrt(C),
                w_o=rng.standard_normal((L + 1, C, C)) / math.sqrt(C),
                w_rbf=rng.standard_normal((R, H)) / math.sqrt(R), w_edge=rng.standard_normal((P, C)))


def test_solid_harmonics_closed_forms():
    x = RNG.standard_normal((40, 3)) * 2.0
    S = edge.solid_sh(x, 3)
    a, b, c = x[:, 0], x[:, 1], x[:, 2]
    r2 = a * a + b * b + c * c
    assert np.allclose(S[:, 0], 1.0)
    assert np.max(np.abs(S[:, 1:4] - math.sqrt(3) * np.stack([b, c, a], 1))) < 1e-13
    s15, s5 = math.sqrt(15), math.sqrt(5)
    want2 = np.stack([s15 * a * b, s15 * b * c, 0.5 * s5 * (3 * c * c - r2), s15 * a * c, 0.5 * s15 * (a * a - b * b)], 1)
    assert np.max(np.abs(S[:, 4:9] - want2)) < 1e-12
    for l in range(4):
        sl = slice(l * l, (l + 1) ** 2)
        assert np.max(np.abs(edge.solid_sh(2.5 * x, 3)[:, sl] - 2.5 ** l * S[:, sl])) < 1e-9 * (1 + np.abs(S).max())
        assert np.max(np.abs(edge.solid_sh(-x, 3)[:, sl] - (-1) ** l * S[:, sl])) < 1e-12
    z = edge.solid_sh(np.zeros((1, 3)), 3)[0]
    assert z[0] == 1.0 and np.all(z[1:] == 0.0)


@pytest.mark.parametrize("L", [1, 2])
def test_edge_form_is_translation_invariant(L):
    p = _weights(40, 16, 2, 6, L, 10 + L)
    rows = layer.neighbors(p["pos"], 3.0)
    a = edge.edge_forward(**p, lmax=L, heads=2, cutoff=3.0, rows=rows)
    q = dict(p, pos=p["pos"] + np.array([17.25, -5.125, 2.0]))
    b = edge.edge_forward(**q, lmax=L, heads=2, cutoff=3.0, rows=rows)
    rms = np.sqrt(np.mean(a["out"] ** 2))
    assert rms > 0 and np.max(np.abs(a["out"] - b["out"])) / rms < 1e-12


@pytest.mark.parametrize("L", [1, 2, 3])
def test_edge_form_is_rotation_equivariant(L):
    p = _weights(36, 8, 2, 5, L, 20 + L)
    rows = layer.neighbors(p["pos"], 3.0)
    base = edge.edge_forward(**p, lmax=L, heads=2, cutoff=3.0, rows=rows)
    R = so3.rotation_matrix(0.4, 2.1, -1.3)
    D = so3.wigner_d_blocks(R, L)
    rot = dict(p, pos=p["pos"] @ R.T, h=np.einsum("ab,nbc->nac", D, p["h"]))
    o = edge.edge_forward(**rot, lmax=L, heads=2, cutoff=3.0, rows=rows)
    want = np.einsum("ab,nbc->nac", D, base["out"])
    assert np.max(np.abs(o["out"] - want)) / np.sqrt(np.mean(want ** 2)) < 1e-10


def test_l1_paths_by_hand():
    """Two atoms, each the other's only neighbour (alpha = 1), l_max = 1, one path
    weighted at a time: with x = (r_j - r_i) / r_c and v in (y, z, x) order,
    (0,0,0): m^0 = w v^0;  (0,1,1): m^1 = w v^0 sqrt(3) x;  (1,0,1): m^1 = w v^1;
    (1,1,0): m^0 = -w v^1 . x;  (1,1,1): m^1 = w sqrt(3/2) v^1 x x."""
    C, L, rc = 4, 1, 3.0
    p = _weights(2, C, 1, 4, L, 33)
    p["pos"] = np.array([[0.25, -0.5, 0.75], [1.0, 0.5, -0.25]])
    p["w_v"] = np.broadcast_to(np.eye(C), (L + 1, C, C)).copy()
    p["w_o"] = p["w_v"].copy()
    rows = [np.array([1]), np.array([0])]
    paths = [tuple(t) for t in so3.paths(L)]
    w = RNG.standard_normal(C)
    for t in range(2):
        i, j = t, 1 - t
        x = (p["pos"][j] - p["pos"][i]) / rc
        xv = x[[1, 2, 0]]                                         # (y, z, x)
        v0, v1 = p["h"][j, 0, :], p["h"][j, 1:4, :]               # W_V = I
        want = {(0, 0, 0): (0, w * v0), (0, 1, 1): (1, w * v0 * math.sqrt(3) * xv[:, None]),
                (1, 0, 1): (1, w * v1), (1, 1, 0): (0, -w * np.einsum("a,ac->c", xv, v1)),
                (1, 1, 1): (1, w * math.sqrt(1.5) * np.cross(v1[[2, 0, 1]].T, x).T[[1, 2, 0]])}
        for path, (lo, val) in want.items():
            we = np.zeros((len(paths), C))
            we[paths.index(path)] = w
            m = edge.edge_forward(**dict(p, w_edge=we), lmax=L, heads=1, cutoff=rc, rows=rows)["m"][t]
            blk = m[lo * lo:(lo + 1) ** 2]
            assert np.max(np.abs(blk - np.reshape(val, blk.shape))) < 1e-13, (t, path)
            assert np.max(np.abs(np.delete(m, np.arange(lo * lo, (lo + 1) ** 2), axis=0))) == 0.0


def test_attention_weights_and_coincident_atoms():
    """W_Q = W_K = 0: alpha is the softmax of the distance bias alone, written out here
    for a target with two neighbours; a neighbour at the target's own position has
    S^{l>0} = 0, so only its l_f = 0 paths contribute."""
    C, H, R, L, rc = 4, 1, 5, 1, 3.0
    p = _weights(3, C, H, R, L, 44)
    p["pos"] = np.array([[0.0, 0.0, 0.0], [1.2, 0.0, 0.0], [0.0, 0.0, 0.0]])
    p["w_q"] = np.zeros((C, C))
    p["w_k"] = np.zeros((C, C))
    rows = [np.array([1, 2]), np.array([0]), np.array([0])]
    o = edge.edge_forward(**p, lmax=L, heads=H, cutoff=rc, rows=rows)
    delta = rc / (R - 1)
    b = lambda d: (0.5 * (math.cos(math.pi * d / rc) + 1.0)
                   * sum(p["w_rbf"][k, 0] * math.exp(-((d - k * delta) ** 2) / (2 * delta * delta)) for k in range(R)))
    a1 = math.exp(b(1.2)) / (math.exp(b(1.2)) + math.exp(b(0.0)))
    v = np.concatenate([p["h"][:, :1, :] @ p["w_v"][0], p["h"][:, 1:, :] @ p["w_v"][1]], axis=1)
    S1 = edge.solid_sh(np.array([[1.2 / rc, 0, 0]]), L)
    e1 = edge.edge_product(v[1:2], S1, p["w_edge"], L)[0]
    e2 = edge.edge_product(v[2:3], edge.solid_sh(np.zeros((1, 3)), L), p["w_edge"], L)[0]
    assert np.max(np.abs(o["m"][0] - (a1 * e1 + (1 - a1) * e2))) < 1e-13
    paths = [tuple(t) for t in so3.paths(L)]
    only_lf0 = np.zeros_like(p["w_edge"])
    for q_, (li, lf, lo) in enumerate(paths):
        if lf == 0:
            only_lf0[q_] = p["w_edge"][q_]
    assert np.max(np.abs(e2 - edge.edge_product(v[2:3], S1, only_lf0, L)[0])) < 1e-14
