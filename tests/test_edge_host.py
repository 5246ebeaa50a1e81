"""The library's tables for the exact edge-equivalent form, checked on the CPU
against the oracle's edge-by-edge definition: the node-centric evaluation (each
source coupled with S of its position relative to an origin, the rows summed
with alpha, each target coupled with S of its own position through the
library's addition-theorem x 6j coefficients) must reproduce
sum_j alpha_ij sum_p w_e[p] (v_j (x) S((r_j - r_i) / r_c))_p for any origin.
No GPU: the library's host tables only."""
import ctypes
import math

import numpy as np
import pytest

from atomistic_attention_amd import binding as B
from oracle import edge, layer, so3


@pytest.fixture(scope="module")
def lib():
    return B.load()


def _tables(lib, L, which):
    n = lib.e2v2_edge_coefficients(L, which, None, None, 0)
    assert n > 0
    idx = np.zeros((n, 4), dtype=np.int32)
    val = np.zeros(n, dtype=np.float64)
    got = lib.e2v2_edge_coefficients(L, which, idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     val.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n)
    assert got == n
    return idx, val


def _node_centric(lib, L, pos, v, w_e, rows, rc, origin):
    blocks, _ = _tables(lib, L, 2)
    ng = int(blocks[-1, 3] + 2 * blocks[-1, 2] + 1)
    si, sv = _tables(lib, L, 0)
    ti, tv = _tables(lib, L, 1)
    n, nc, C = v.shape
    Sx = edge.solid_sh((pos - origin) / rc, L)
    G = np.zeros((n, ng, C))
    for (ei, el, eg, _), val in zip(si, sv):
        G[:, eg, :] += val * v[:, ei, :] * Sx[:, el][:, None]
    m = np.zeros((len(rows), nc, C))
    for t, r in enumerate(rows):
        if len(r) == 0:
            continue
        M = G[np.asarray(r)].mean(axis=0)                 # uniform alpha
        Sy = edge.solid_sh((origin - pos[t])[None] / rc, L)[0]
        for (p, eg, em, eo), val in zip(ti, tv):
            m[t, eo, :] += val * w_e[p] * M[eg, :] * Sy[em]
    return m


@pytest.mark.parametrize("L", [0, 1, 2])
def test_node_centric_tables_reproduce_the_edge_form(lib, L):
    rng = np.random.default_rng(70 + L)
    n, C, rc = 30, 3, 2.5
    pos = rng.uniform(-3, 3, (n, 3))
    h = rng.standard_normal((n, (L + 1) ** 2, C))
    P = len(so3.paths(L))
    w_e = rng.standard_normal((P, C))
    rows = layer.neighbors(pos, rc)
    eye = np.broadcast_to(np.eye(C), (L + 1, C, C)).copy()
    # W_Q = W_K = W_rbf = 0: alpha is uniform over each row, as _node_centric takes it
    ref = edge.edge_forward(pos, h, np.zeros((C, C)), np.zeros((C, C)), eye, eye, np.zeros((4, 1)), w_e, lmax=L,
                            heads=1, cutoff=rc, rows=rows)["m"]
    scale = np.sqrt(np.mean(ref ** 2))
    assert scale > 0
    for origin in (0.5 * (pos.min(0) + pos.max(0)), np.array([4.0, -7.5, 2.25]), np.zeros(3)):
        got = _node_centric(lib, L, pos, h, w_e, rows, float(np.float32(rc)), origin)
        assert np.max(np.abs(got - ref)) / scale < 1e-11, origin


def test_edge_tables_sizes_and_errors(lib):
    counts = [[lib.e2v2_edge_coefficients(L, w, None, None, 0) for w in range(3)] for L in range(3)]
    assert counts[2] == [158, 305, 16] and counts[1] == [16, 23, 5] and counts[0] == [1, 1, 1]
    assert lib.e2v2_edge_coefficients(3, 0, None, None, 0) == -1
    assert lib.e2v2_edge_coefficients(2, 3, None, None, 0) == -1
