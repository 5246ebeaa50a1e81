"""Pins of the test-side Hilbert-curve reference (tests/_curve.py), on the CPU.

Properties every 3-D Hilbert curve has, which the GPU order is then compared
against bit for bit: on a full 2^k lattice the curve visits every point once,
each step moves to a face-adjacent point, each aligned run of 8^m consecutive
points fills an aligned 2^m cube, and it starts in the origin's corner.  A Morton
order, a wrong Gray code or a skipped exchange breaks the unit steps."""
import itertools

import numpy as np
import pytest

from tests import _curve


def _lattice(k, spacing=1.0, origin=(0.0, 0.0, 0.0)):
    m = 1 << k
    g = np.array(list(itertools.product(range(m), repeat=3)), dtype=np.int64)
    rng = np.random.default_rng(k)
    g = g[rng.permutation(len(g))]                      # ids carry no order
    return g, (g * spacing + np.asarray(origin)).astype(np.float32)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_lattice_walk_is_a_hilbert_curve(k):
    g, pos = _lattice(k, spacing=1.0, origin=(-3.0, 5.0, 0.5))
    order = _curve.target_order(pos)
    assert np.array_equal(np.sort(order), np.arange(len(g)))
    path = g[order]
    steps = np.abs(np.diff(path, axis=0)).sum(axis=1)
    assert np.all(steps == 1)                            # face-adjacent steps only
    assert np.array_equal(path[0], [0, 0, 0])
    for m in range(1, k):
        blk = path.reshape(-1, 8 ** m, 3)
        lo = blk.min(axis=1)
        assert np.all(blk.max(axis=1) - lo == (1 << m) - 1)
        assert np.all(lo % (1 << m) == 0)


def test_index_is_a_bijection_on_the_grid():
    q = np.array(list(itertools.product(range(8), repeat=3)), dtype=np.int64)
    key = _curve.hilbert_index(q, bits=3)
    assert np.array_equal(np.sort(key), np.arange(512))
    path = q[np.argsort(key)]
    assert np.all(np.abs(np.diff(path, axis=0)).sum(axis=1) == 1)


def test_morton_order_fails_the_step_test():
    """The step test has teeth: Z-order jumps."""
    q = np.array(list(itertools.product(range(4), repeat=3)), dtype=np.int64)
    z = np.zeros(len(q), dtype=np.int64)
    for b in range(2):
        for a in range(3):
            z |= ((q[:, a] >> b) & 1) << (3 * b + (2 - a))
    path = q[np.argsort(z)]
    assert np.any(np.abs(np.diff(path, axis=0)).sum(axis=1) > 1)


def test_cell_grid_rule():
    """Cells of side 2^k: 1,000 atoms in a 20 A cube: V / (8 n) = 1 -> k = 0,
    and a long thin box is capped at 1023 cells along its longest side."""
    rng = np.random.default_rng(0)
    pos = rng.uniform(0, 20, (1000, 3)).astype(np.float32)
    pos[0] = 0.0
    pos[1] = 20.0
    q = _curve.cells(pos)
    assert np.array_equal(q, np.floor(pos).astype(np.int64))
    line = np.zeros((5000, 3), dtype=np.float32)
    line[:, 0] = np.linspace(0, 1e4, 5000, dtype=np.float32)
    q = _curve.cells(line)
    assert q[:, 0].max() < 1023 and q[:, 0].max() > 511
    assert np.all(q[:, 1:] == 0)


def test_degenerate_positions():
    same = np.full((7, 3), 2.5, dtype=np.float32)
    assert np.array_equal(_curve.target_order(same), np.arange(7))
    odd = np.array([[0, 0, 0], [np.nan, 1, 1], [np.inf, 2, 2], [1, 1, 1]], dtype=np.float32)
    o = _curve.target_order(odd)
    assert np.array_equal(np.sort(o), np.arange(4))
