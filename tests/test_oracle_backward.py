"""Pins of the feature-gradient oracle (oracle/backward.py).

The torch fp64 layer is checked against the numpy oracle's forward pass, and
its reverse-mode gradient against central finite differences of the numpy
forward pass (layer.layer_forward), so a dropped term, a wrong sign or a
transposed weight in either place fails here.  Special cases: one neighbour
(softmax weight 1, so q and k receive no gradient), an isolated atom (its
gradient comes only from other targets through it as a source; with no
neighbours on either side it is zero), an atom at the origin (l_f > 0 paths
vanish)."""
import numpy as np
import pytest

from oracle import backward, layer, so3

LMAX, C, HEADS, R, CUT = 2, 16, 2, 8, 3.0


def _system(seed, n=20, side=5.0, extra=()):
    rng = np.random.default_rng(seed)
    pos = rng.uniform(-side / 2, side / 2, (n, 3))
    if extra:
        pos = np.concatenate([pos, np.asarray(extra, dtype=np.float64)], axis=0)
    pos = pos.astype(np.float32).astype(np.float64)
    nc = (LMAX + 1) ** 2
    P = len(so3.paths(LMAX))
    W = dict(
        w_q=rng.standard_normal((C, C)) / np.sqrt(C),
        w_k=rng.standard_normal((C, C)) / np.sqrt(C),
        w_v=rng.standard_normal((LMAX + 1, C, C)) / np.sqrt(C),
        w_o=rng.standard_normal((LMAX + 1, C, C)) / np.sqrt(C),
        w_rbf=rng.standard_normal((R, HEADS)) / np.sqrt(R),
        w_src=rng.standard_normal((P, C)) / np.sqrt(P),
        w_tgt=rng.standard_normal((P, C)) / np.sqrt(P))
    h = rng.standard_normal((pos.shape[0], nc, C))
    g = rng.standard_normal((pos.shape[0], nc, C))
    return pos, h, W, g


def _fwd_np(pos, h, W, rows):
    return layer.layer_forward(pos, h, **W, lmax=LMAX, heads=HEADS, cutoff=CUT, rows=rows)["out"]


def _grad(pos, h, W, g, rows):
    return backward.grad_h(pos, h, **W, g=g, lmax=LMAX, heads=HEADS, cutoff=CUT, rows=rows)


def test_torch_forward_matches_numpy_oracle():
    import torch
    pos, h, W, _ = _system(1, extra=[[0.0, 0.0, 0.0], [40.0, 0.0, 0.0]])
    rows = layer.neighbors(pos, CUT)
    ref = _fwd_np(pos, h, W, rows)
    got = backward.layer_forward_torch(pos, torch.tensor(h), **W, lmax=LMAX, heads=HEADS, cutoff=CUT,
                                       rows=rows).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("seed", [2, 3])
def test_gradient_matches_central_differences(seed):
    """Directional derivatives along random u: (L(h + eps u) - L(h - eps u)) / 2 eps of the
    numpy forward pass against <dL/dh, u>; also along u restricted to the l = 0 block
    (the only block feeding q and k) and to the l = 2 block."""
    pos, h, W, g = _system(seed, extra=[[0.0, 0.0, 0.0]])
    rows = layer.neighbors(pos, CUT)
    assert min(r.size for r in rows[:-1]) >= 1 and max(r.size for r in rows) >= 4
    gr = _grad(pos, h, W, g, rows)
    rng = np.random.default_rng(seed + 100)
    eps = 1e-5
    masks = [np.ones_like(h), np.zeros_like(h), np.zeros_like(h)]
    masks[1][:, 0, :] = 1.0
    masks[2][:, 4:9, :] = 1.0
    for mk in masks:
        u = rng.standard_normal(h.shape) * mk
        lp = np.sum(g * _fwd_np(pos, h + eps * u, W, rows))
        lm = np.sum(g * _fwd_np(pos, h - eps * u, W, rows))
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(gr * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_single_entries_by_central_differences():
    """Element-wise finite differences on a few entries of l = 0, 1, 2 at several atoms."""
    pos, h, W, g = _system(4)
    rows = layer.neighbors(pos, CUT)
    gr = _grad(pos, h, W, g, rows)
    eps = 1e-5
    for (a, e, c) in [(0, 0, 3), (5, 0, 15), (7, 2, 0), (11, 6, 9), (19, 8, 7)]:
        d = np.zeros_like(h)
        d[a, e, c] = eps
        fd = (np.sum(g * _fwd_np(pos, h + d, W, rows)) - np.sum(g * _fwd_np(pos, h - d, W, rows))) / (2 * eps)
        assert abs(fd - gr[a, e, c]) <= 1e-7 * max(1.0, abs(gr[a, e, c])), (a, e, c, fd, gr[a, e, c])


def test_one_neighbour_pair_has_no_query_key_gradient():
    """Two atoms within the cutoff, each the other's only neighbour: the softmax
    weight is 1 whatever q and k are, so the gradient does not depend on W_Q, W_K,
    and equals that with W_Q = W_K = 0."""
    pos, h, W, g = _system(5, n=0, extra=[[0.3, -0.2, 0.1], [1.1, 0.4, -0.9]])
    rows = layer.neighbors(pos, CUT)
    assert [r.tolist() for r in rows] == [[1], [0]]
    g1 = _grad(pos, h, W, g, rows)
    W0 = dict(W, w_q=np.zeros((C, C)), w_k=np.zeros((C, C)))
    g0 = _grad(pos, h, W0, g, rows)
    assert np.max(np.abs(g1 - g0)) <= 1e-13 * np.max(np.abs(g1))
    assert np.max(np.abs(g1)) > 0


def test_isolated_atom_has_zero_gradient():
    pos, h, W, g = _system(6, extra=[[50.0, 50.0, 50.0]])
    rows = layer.neighbors(pos, CUT)
    assert rows[-1].size == 0
    gr = _grad(pos, h, W, g, rows)
    assert np.all(gr[-1] == 0.0)
    assert np.max(np.abs(gr[:-1])) > 0


def test_sampled_targets_give_the_full_gradient_at_sampled_atoms():
    """B2: with targets = sample plus every member of the sample's rows, the
    gradient at the sampled atoms equals the whole-system gradient."""
    pos, h, W, g = _system(7, n=40, side=6.0)
    rows = layer.neighbors(pos, CUT)
    full = _grad(pos, h, W, g, rows)
    sample = np.array([3, 17, 29])
    tg = np.unique(np.concatenate([sample] + [rows[a] for a in sample]))
    assert tg.size < pos.shape[0]
    got = backward.grad_h(pos, h, **W, g=g[tg], lmax=LMAX, heads=HEADS, cutoff=CUT, rows=[rows[t] for t in tg],
                          targets=tg)
    assert np.max(np.abs(got[sample] - full[sample])) <= 1e-12 * np.max(np.abs(full))
    other = np.setdiff1d(np.arange(pos.shape[0]), tg)
    assert np.max(np.abs(got[other] - full[other])) > 1e-6      # elsewhere the sample is incomplete


# ---------------------------------------------------------------- B3: positions

def _gpos(pos, h, W, g, rows, lmax=LMAX):
    return backward.grad_pos_h(pos, h, **W, g=g, lmax=lmax, heads=HEADS, cutoff=CUT, rows=rows)[0]


@pytest.mark.parametrize("seed", [12, 13])
def test_position_gradient_matches_central_differences(seed):
    """Directional and element-wise derivatives of the numpy forward pass in the
    positions (lists held fixed) against dL/dpos."""
    pos, h, W, g = _system(seed)
    rows = layer.neighbors(pos, CUT)
    gp = _gpos(pos, h, W, g, rows)
    rng = np.random.default_rng(seed + 7)
    eps = 1e-6
    L = lambda p: np.sum(g * _fwd_np(p, h, W, rows))
    u = rng.standard_normal(pos.shape)
    fd = (L(pos + eps * u) - L(pos - eps * u)) / (2 * eps)
    an = float(np.sum(gp * u))
    assert abs(fd - an) <= 2e-6 * max(1.0, abs(an)), (fd, an)
    for a, k in [(0, 0), (4, 1), (9, 2), (15, 0)]:
        d = np.zeros_like(pos)
        d[a, k] = eps
        fd = (L(pos + d) - L(pos - d)) / (2 * eps)
        assert abs(fd - gp[a, k]) <= 2e-6 * max(1.0, abs(gp[a, k])), (a, k, fd, gp[a, k])


def test_position_gradient_on_a_list_with_pairs_beyond_the_cutoff():
    """A reused list (Tessera article, neighbour reuse) holds pairs that have moved
    past r_c.  Their bias and its slope are 0 (the cutoff mask), so the torch
    gradient must still match central differences of the numpy forward pass; a
    slope term left on those pairs, or a missing one below r_c, fails here."""
    pos, h, W, g = _system(14)
    rows = layer.neighbors(pos, CUT + 0.6)               # the list of a larger radius
    far = sum(int(np.sum(np.linalg.norm(pos[r] - pos[i], axis=1) >= CUT)) for i, r in enumerate(rows))
    assert far >= 20
    gp = _gpos(pos, h, W, g, rows)
    rng = np.random.default_rng(21)
    eps = 1e-6
    L = lambda p: np.sum(g * _fwd_np(p, h, W, rows))
    for _ in range(2):
        u = rng.standard_normal(pos.shape)
        fd = (L(pos + eps * u) - L(pos - eps * u)) / (2 * eps)
        an = float(np.sum(gp * u))
        assert abs(fd - an) <= 2e-6 * max(1.0, abs(an)), (fd, an)


def test_position_gradient_vanishes_without_geometry():
    """l_max = 0 and W_rbf = 0: the output does not depend on the positions."""
    pos, h, W, g = _system(14)
    nc = 1
    P = len(so3.paths(0))
    W0 = dict(W, w_v=W["w_v"][:1], w_o=W["w_o"][:1], w_src=W["w_src"][:P], w_tgt=W["w_tgt"][:P],
              w_rbf=np.zeros_like(W["w_rbf"]))
    rows = layer.neighbors(pos, CUT)
    gp = _gpos(pos, h[:, :nc], W0, g[:, :nc], rows, lmax=0)
    assert np.all(gp == 0.0)


def test_bias_only_gradient_is_translation_and_rotation_invariant():
    """l_max = 0: positions enter through pair distances only, so the gradient sums
    to zero (no net force) and has no net torque."""
    pos, h, W, g = _system(15)
    P = len(so3.paths(0))
    W0 = dict(W, w_v=W["w_v"][:1], w_o=W["w_o"][:1], w_src=W["w_src"][:P], w_tgt=W["w_tgt"][:P])
    rows = layer.neighbors(pos, CUT)
    gp = _gpos(pos, h[:, :1], W0, g[:, :1], rows, lmax=0)
    scale = np.max(np.abs(gp))
    assert scale > 1e-3
    assert np.max(np.abs(gp.sum(axis=0))) <= 1e-12 * scale * pos.shape[0]
    assert np.max(np.abs(np.cross(pos, gp).sum(axis=0))) <= 1e-12 * scale * pos.shape[0] * 5


def test_position_gradient_finite_with_an_atom_at_the_origin():
    """B3: the atom at the origin gets a finite gradient (bias terms only, its
    encoding held constant), and every other atom's gradient still matches
    central differences."""
    pos, h, W, g = _system(16, extra=[[0.0, 0.0, 0.0]])
    rows = layer.neighbors(pos, CUT)
    assert rows[-1].size > 0
    gp = _gpos(pos, h, W, g, rows)
    assert np.all(np.isfinite(gp))
    eps = 1e-6
    L = lambda p: np.sum(g * _fwd_np(p, h, W, rows))
    u = np.random.default_rng(3).standard_normal(pos.shape)
    u[-1] = 0.0
    fd = (L(pos + eps * u) - L(pos - eps * u)) / (2 * eps)
    an = float(np.sum(gp * u))
    assert abs(fd - an) <= 2e-6 * max(1.0, abs(an)), (fd, an)


def test_stack_gradient_matches_central_differences():
    """B4: the gradients of a two-layer stack (5 A and 8 A lists, the second taken
    from a capped list) against central differences of the numpy layer
    composition over the same fixed lists, in h and in pos."""
    import dataclasses
    from atomistic_attention_amd import workloads as W
    from oracle import stack as OS
    cfg = dataclasses.replace(W.STACKS["s1"], n=48, steps=1, cutoffs=(5.0, 8.0), max_neighbors=20)
    st = W.make_stack(cfg)
    pos, h0 = st.traj[0], st.h0
    state = OS.StackState([wl.cfg.cutoff for wl in st.layers], cfg.max_neighbors)
    state.rebuild(pos, 0)
    rng = np.random.default_rng(21)
    g = rng.standard_normal(h0.shape)
    gp, gh = backward.stack_grad_pos_h(pos, h0, st.layers, state.rows, g)

    def L(p, h):
        x = h
        for wl in st.layers:
            c = wl.cfg
            x = layer.layer_forward(p, x, wl.w_q, wl.w_k, wl.w_v, wl.w_o, wl.w_rbf, wl.w_src, wl.w_tgt, lmax=c.lmax,
                                    heads=c.heads, cutoff=c.cutoff, rows=state.rows[float(np.float32(c.cutoff))])["out"]
        return float(np.sum(g * x))

    eps = 1e-6
    u = rng.standard_normal(h0.shape)
    fd = (L(pos, h0 + eps * u) - L(pos, h0 - eps * u)) / (2 * eps)
    assert abs(fd - np.sum(gh * u)) <= 1e-6 * max(1.0, abs(fd)), (fd, np.sum(gh * u))
    v = rng.standard_normal(pos.shape)
    fd = (L(pos + eps * v, h0) - L(pos - eps * v, h0)) / (2 * eps)
    assert abs(fd - np.sum(gp * v)) <= 2e-6 * max(1.0, abs(fd)), (fd, np.sum(gp * v))


def test_stack_gradient_with_bf16_rounding_between_layers_is_the_chain_rule():
    """B4 with bf16 storage: the stack gradient with rounding between layers equals
    the chain rule written out with separate one-layer gradients -- the second
    layer's vector-Jacobian product at the rounded first output (B3), then the
    first layer's at h0 with that result -- and the rounding changes the gradient
    (it is not silently skipped)."""
    import dataclasses
    import torch
    from atomistic_attention_amd import workloads as W
    from oracle import stack as OS
    cfg = dataclasses.replace(W.STACKS["s1"], n=40, steps=1, cutoffs=(5.0, 8.0), max_neighbors=0)
    st = W.make_stack(cfg)
    pos, h0 = st.traj[0], st.h0
    state = OS.StackState([wl.cfg.cutoff for wl in st.layers], 0)
    state.rebuild(pos, 0)
    rows = lambda wl: state.rows[float(np.float32(wl.cfg.cutoff))]
    g = np.random.default_rng(22).standard_normal(h0.shape)
    gp, gh = backward.stack_grad_pos_h(pos, h0, st.layers, state.rows, g, round_between=True)
    gp0, gh0 = backward.stack_grad_pos_h(pos, h0, st.layers, state.rows, g)
    l1, l2 = st.layers
    kw = lambda wl: dict(w_q=wl.w_q, w_k=wl.w_k, w_v=wl.w_v, w_o=wl.w_o, w_rbf=wl.w_rbf, w_src=wl.w_src,
                         w_tgt=wl.w_tgt, lmax=wl.cfg.lmax, heads=wl.cfg.heads, cutoff=wl.cfg.cutoff, rows=rows(wl))
    x1 = layer.layer_forward(pos, h0, **kw(l1))["out"]
    x1r = OS._round_bf16(x1)
    assert np.max(np.abs(x1r - x1)) > 0
    p2, d1 = backward.grad_pos_h(pos, x1r, g=g, **kw(l2))              # layer 2 at its rounded input
    p1, d0 = backward.grad_pos_h(pos, h0, g=d1, **kw(l1))              # layer 1 with layer 2's dL/dx1
    assert np.max(np.abs(gh - d0)) <= 1e-10 * np.max(np.abs(d0))
    assert np.max(np.abs(gp - (p1 + p2))) <= 1e-10 * np.max(np.abs(p1 + p2))
    assert np.max(np.abs(gh - gh0)) > 1e-6 * np.max(np.abs(gh0))
