"""Pins of the stack oracle (oracle/stack.py): list filtering against the brute
force search at the smaller cutoff, the rebuild rule on trajectories whose
rebuild steps are known in advance, exact displacement arithmetic, topology
reuse, and rotation equivariance of the whole stack."""
import dataclasses

import numpy as np
import pytest

from atomistic_attention_amd import workloads as W
from oracle import layer, so3, stack

RNG = np.random.default_rng(2024)


def _pts(n, side):
    return RNG.uniform(-side / 2, side / 2, (n, 3)).astype(np.float32).astype(np.float64)


def test_filter_equals_search_at_smaller_cutoff():
    """Filtering the 8 A list (uncapped, and capped where the cap does not bind
    inside 5 A) gives exactly the brute-force 5 A list, order included."""
    pos = _pts(1500, 25.0)
    big = layer.neighbors(pos, 8.0)
    small = layer.neighbors(pos, 5.0)
    got = stack.filter_rows(pos, big, 5.0)
    assert all(np.array_equal(a, b) for a, b in zip(got, small))
    capped = layer.neighbors(pos, 8.0, 120)
    assert max(r.size for r in small) < 120
    got = stack.filter_rows(pos, capped, 5.0)
    assert all(np.array_equal(a, b) for a, b in zip(got, small))


def test_filter_drops_invalid_and_keeps_order():
    pos = np.array([[0, 0, 0], [1, 0, 0], [0, 2, 0], [0, 0, 6]], dtype=np.float64)
    rows = [np.array([3, -1, 2, 1, 7], dtype=np.int32), np.array([0], dtype=np.int32),
            np.array([], dtype=np.int32), np.array([0, 1], dtype=np.int32)]
    got = stack.filter_rows(pos, rows, 5.0)
    assert got[0].tolist() == [2, 1] and got[1].tolist() == [0] and got[2].size == 0 and got[3].size == 0


def test_displacement_exact_and_strict():
    """Dyadic coordinates make every displacement exact: a move of exactly 0.25 A
    does not trigger (the rule is 'more than'), 0.25 + 2^-10 does."""
    ref = np.array([[1.0, 2.0, 3.0], [-4.0, 0.5, 0.25]])
    p = ref.copy()
    p[1, 0] += 0.25
    assert stack.max_displacement2(p, ref) == 0.0625
    st = stack.StackState([5.0, 8.0], 0)
    st.ref, st.since = ref, 3
    assert not st.need_rebuild(p)
    p[1, 0] += 2.0 ** -10
    assert st.need_rebuild(p)
    p[0, 2] = np.nan
    assert stack.max_displacement2(p, ref) == np.inf


def _tiny_stack(steps, jumps=(), storage="fp32"):
    cfg = dataclasses.replace(W.STACKS["s1"], n=64, steps=steps, sigma=0.002)
    st = W.make_stack(cfg, jumps=jumps)
    if storage != st.base.storage:
        st.layers = [dataclasses.replace(wl, cfg=dataclasses.replace(wl.cfg, storage=storage)) for wl in st.layers]
    return st


@pytest.mark.parametrize("jumps,want", [((), [0, 10, 20]),
                                        (((4, 5, (0.3, 0.0, 0.0)),), [0, 4, 14, 24]),
                                        (((6, 9, (0.0, 0.26, 0.0)), (7, 2, (0.0, 0.0, -0.3))), [0, 6, 7, 17])])
def test_rebuild_schedule(jumps, want):
    """Every 10 steps, and at once after a move of more than 0.25 A (a 0.002 A random
    walk reaches nowhere near it in 25 steps)."""
    st = _tiny_stack(25, jumps)
    state = stack.StackState([5.0, 5.0, 5.0, 8.0], 256)
    for t, p in enumerate(st.traj):
        if state.need_rebuild(p):
            state.rebuild(p, t)
        state.since += 1
    assert state.rebuilds == want


def test_topology_reused_between_rebuilds():
    """Two atoms 4.9 A apart, then 5.05 A after a 0.21 A move off the axis: the 5 A
    layers keep the pair (positions updated, topology kept; with one neighbour the
    new direction changes the output) until the 10-step rebuild drops it."""
    base = _tiny_stack(1)
    pos0 = np.array([[0.0, 0.0, 0.0], [4.9, 0.0, 0.0]])
    pos1 = np.array([[0.0, 0.0, 0.0], [5.05, 0.15, 0.0]])
    layers = [dataclasses.replace(wl, cfg=dataclasses.replace(wl.cfg, n=2)) for wl in base.layers[:3]]
    h0 = RNG.standard_normal((2, 9, 32))
    state = stack.StackState([5.0] * 3, 0)
    o0 = stack.stack_step(state, pos0, h0, layers, 0, "fp32")
    o1 = stack.stack_step(state, pos1, h0, layers, 1, "fp32")
    assert state.rebuilds == [0] and state.rows[5.0][0].tolist() == [1]
    assert np.abs(o1).max() > 0.0 and np.abs(o1 - o0).max() > 0.0   # same pair, new distance
    for t in range(2, 10):
        stack.stack_step(state, pos1, h0, layers, t, "fp32")
    o10 = stack.stack_step(state, pos1, h0, layers, 10, "fp32")
    assert state.rebuilds == [0, 10] and state.rows[5.0][0].size == 0
    assert np.abs(o10).max() == 0.0                                  # no neighbours: m = 0, out = 0


def test_stack_rotation_equivariance():
    """Rotating the whole trajectory by R rotates every step's stack output by D(R)
    (fp64 between layers, lists taken from the unrotated run once the rotated
    search is seen to agree)."""
    st = _tiny_stack(4, ((2, 3, (0.3, 0.0, 0.0)),), storage="fp64")
    L = st.base.lmax
    outs, rb = stack.run_stack(st)
    assert rb == [0, 2]
    R = so3.rotation_matrix(0.7, 1.9, -0.4)
    D = so3.wigner_d_blocks(R, L)
    state = stack.StackState([wl.cfg.cutoff for wl in st.layers], st.cfg.max_neighbors)
    ref_state = stack.StackState([wl.cfg.cutoff for wl in st.layers], st.cfg.max_neighbors)
    h0r = np.einsum("ab,nbc->nac", D, st.h0)
    for t, p in enumerate(st.traj):
        pr = p @ R.T
        if ref_state.need_rebuild(p):
            ref_state.rebuild(p, t)
        ref_state.since += 1
        if state.need_rebuild(pr):
            state.rebuild(pr, t)
            for c, rows in state.rows.items():
                assert all(np.array_equal(a, b) for a, b in zip(rows, ref_state.rows[c]))
            state.rows = ref_state.rows
        o = stack.stack_step(state, pr, h0r, st.layers, t, "fp64")
        want = np.einsum("ab,nbc->nac", D, outs[t])
        assert np.max(np.abs(o - want)) / np.sqrt(np.mean(outs[t] ** 2)) < 1e-10
    assert state.rebuilds == rb


def test_one_layer_stack_is_the_layer():
    st = _tiny_stack(1)
    wl = st.layers[3]
    state = stack.StackState([8.0], 256)
    o = stack.stack_step(state, st.traj[0], st.h0, [wl], 0, "fp32")
    ref = layer.layer_forward(st.traj[0], st.h0, wl.w_q, wl.w_k, wl.w_v, wl.w_o, wl.w_rbf, wl.w_src, wl.w_tgt,
                              lmax=wl.cfg.lmax, heads=wl.cfg.heads, cutoff=8.0, max_neighbors=256)["out"]
    assert np.array_equal(o, ref)
