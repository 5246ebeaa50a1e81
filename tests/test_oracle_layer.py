"""Pins of the oracle's layer (neighbours, distance bias, attention, whole layer)
against library routines (scipy cKDTree, torch scaled_dot_product_attention),
closed-form values, special cases and rotation equivariance."""
import math

import numpy as np
import pytest
import torch
from scipy.spatial import cKDTree

from atomistic_attention_amd import workloads as W
from oracle import layer, so3

RNG = np.random.default_rng(77)


def _pts(n, side):
    return RNG.uniform(-side / 2, side / 2, (n, 3)).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------- O1 neighbours
def test_neighbors_match_kdtree_and_numpy():
    pos = _pts(3000, 30.0)
    rc = 4.0
    rows = layer.neighbors(pos, rc)
    tree = cKDTree(pos)
    ref = tree.query_ball_point(pos, rc)
    for i, (a, b) in enumerate(zip(rows, ref)):
        b = np.sort([j for j in b if j != i])
        assert np.array_equal(a, b), i
    rows_np = layer.neighbors_numpy(pos, rc, targets=np.arange(0, 3000, 7))
    for t, i in enumerate(range(0, 3000, 7)):
        assert np.array_equal(rows_np[t], rows[i])


def test_neighbors_capped_keep_nearest():
    pos = _pts(2000, 18.0)
    rc, K = 5.0, 40
    rows = layer.neighbors(pos, rc, K)
    full = layer.neighbors(pos, rc, 0)
    d, j = cKDTree(pos).query(pos, k=K + 1)
    over = 0
    for i in range(pos.shape[0]):
        if full[i].size <= K:
            assert np.array_equal(rows[i], full[i])
        else:
            over += 1
            assert rows[i].size == K
            assert np.array_equal(rows[i], np.sort(j[i, 1:]))
            assert np.all(np.diff(rows[i]) > 0)
    assert over > 100


def test_neighbors_exclude_self_and_empty():
    pos = np.array([[0, 0, 0], [1, 0, 0], [50, 0, 0]], dtype=np.float64)
    rows = layer.neighbors(pos, 2.0)
    assert [r.tolist() for r in rows] == [[1], [0], []]


def test_neighbor_predicate_is_strict():
    # d = 2 exactly (representable) is not inside a cutoff of 2
    pos = np.array([[0, 0, 0], [2, 0, 0], [0, 1.5, 0]], dtype=np.float64)
    rows = layer.neighbors(pos, 2.0)
    assert rows[0].tolist() == [2]


# ---------------------------------------------------------------- O6 distance bias
def test_rbf_bias_closed_values():
    rc, R = 6.0, 7
    delta = rc / (R - 1)
    eye = np.eye(R)
    mu = np.arange(R) * delta
    b = layer.rbf_bias(mu, eye, rc)                    # b[k, h] = f_c(mu_k) phi_h(mu_k)
    fc = 0.5 * (np.cos(np.pi * mu / rc) + 1)
    assert np.allclose(np.diag(b), fc, atol=1e-15)     # phi_k(mu_k) = 1
    assert abs(layer.rbf_bias(np.array(0.0), eye, rc)[0] - 1.0) < 1e-15            # f_c(0) = 1
    assert abs(layer.rbf_bias(np.array(rc / 2), eye, rc)[3] - 0.5) < 1e-15         # f_c(rc/2) = 1/2, mu_3 = rc/2
    assert np.max(np.abs(layer.rbf_bias(np.array(rc), eye, rc))) < 1e-15           # f_c(rc) = 0
    d = mu[2] + delta
    v = layer.rbf_bias(np.array(d), eye, rc)[2] / (0.5 * (math.cos(math.pi * d / rc) + 1))
    assert abs(v - math.exp(-0.5)) < 1e-15                                          # one width away


# ---------------------------------------------------------------- O6 attention
def _rand_layer(n, C, H, R, L, side, seed):
    rng = np.random.default_rng(seed)
    npath = len(so3.paths(L))
    nc = (L + 1) ** 2
    return dict(
        pos=rng.uniform(-side / 2, side / 2, (n, 3)).astype(np.float32).astype(np.float64),
        h=rng.standard_normal((n, nc, C)),
        w_q=rng.standard_normal((C, C)) / math.sqrt(C), w_k=rng.standard_normal((C, C)) / math.sqrt(C),
        w_v=rng.standard_normal((L + 1, C, C)) / math.sqrt(C), w_o=rng.standard_normal((L + 1, C, C)) / math.sqrt(C),
        w_rbf=rng.standard_normal((R, H)), w_src=rng.standard_normal((npath, C)),
        w_tgt=rng.standard_normal((npath, C)))


def test_lmax0_is_sparse_multihead_attention():
    """At l_max = 0 every tensor product is a per-channel scale, so the layer is plain
    multi-head attention with an additive distance bias over the neighbour mask:
    checked against torch's scaled_dot_product_attention with a dense mask."""
    n, C, H, R, rc = 48, 16, 2, 6, 6.0
    p = _rand_layer(n, C, H, R, 0, 12.0, 5)
    o = layer.layer_forward(**p, lmax=0, heads=H, cutoff=rc)
    rows = o["rows"]
    assert all(r.size > 0 for r in rows)
    d_head = C // H
    pos, h0 = p["pos"], p["h"][:, 0, :]
    q = torch.tensor(h0 @ p["w_q"]).view(n, H, d_head).transpose(0, 1)
    k = torch.tensor(h0 @ p["w_k"]).view(n, H, d_head).transpose(0, 1)
    v = torch.tensor((h0 @ p["w_v"][0]) * p["w_src"][0]).view(n, H, d_head).transpose(0, 1)
    mask = torch.full((H, n, n), -math.inf, dtype=torch.float64)
    for i, js in enumerate(rows):
        d = np.linalg.norm(pos[js] - pos[i], axis=1)
        mask[:, i, js] = torch.tensor(layer.rbf_bias(d, p["w_rbf"], rc).T)
    att = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    m_ref = att.transpose(0, 1).reshape(n, C).numpy()
    assert np.max(np.abs(o["m"][:, 0, :] - m_ref)) < 1e-12
    out_ref = (m_ref * p["w_tgt"][0]) @ p["w_o"][0]
    assert np.max(np.abs(o["out"][:, 0, :] - out_ref)) < 1e-12


def test_single_neighbour_and_empty_set():
    p = _rand_layer(3, 8, 1, 4, 2, 1.0, 9)
    p["pos"] = np.array([[0.3, 0.1, 0.2], [1.0, -0.4, 0.7], [40.0, 0, 0]])
    o = layer.layer_forward(**p, lmax=2, heads=1, cutoff=3.0)
    hp = {int(s): o["hprime"][t] for t, s in enumerate(o["src"])}
    assert np.max(np.abs(o["m"][0] - hp[1])) < 1e-14      # alpha = 1
    assert np.max(np.abs(o["m"][1] - hp[0])) < 1e-14
    assert np.all(o["m"][2] == 0) and np.all(o["out"][2] == 0)


def test_equal_logits_give_mean():
    n, C, H, L = 7, 8, 2, 2
    p = _rand_layer(n, C, H, 5, L, 1.0, 11)
    dirs = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [-1, 0, 0], [0, -1, 0], [0, 0, -1]], dtype=float)
    p["pos"] = np.vstack([[0, 0, 0], 2.0 * dirs])
    p["h"][1:, 0, :] = p["h"][1, 0, :]                     # identical k rows
    o = layer.layer_forward(**p, lmax=L, heads=H, cutoff=2.5)
    hp = o["hprime"][[list(o["src"]).index(j) for j in range(1, 7)]]
    assert np.max(np.abs(o["m"][0] - hp.mean(axis=0))) < 1e-14


# ---------------------------------------------------------------- whole layer
@pytest.mark.parametrize("L", [1, 2, 3])
def test_layer_rotation_equivariance(L):
    """Rotating positions by R and features by D(R) rotates the output by D(R)."""
    n, C, H = 90, 16, 2
    p = _rand_layer(n, C, H, 6, L, 9.5, 100 + L)
    rc = 4.0
    base = layer.layer_forward(**p, lmax=L, heads=H, cutoff=rc)
    for trial in range(2):
        R = so3.rotation_matrix(*np.random.default_rng(trial).uniform(0, 3, 3))
        D = so3.wigner_d_blocks(R, L)
        rot = dict(p)
        rot["pos"] = p["pos"] @ R.T
        rot["h"] = np.einsum("ab,nbc->nac", D, p["h"])
        rows_rot = layer.neighbors_numpy(rot["pos"], rc)   # fp64 search on the rotated set
        assert all(np.array_equal(a, b) for a, b in zip(rows_rot, base["rows"]))
        o = layer.layer_forward(**rot, lmax=L, heads=H, cutoff=rc, rows=base["rows"])
        want = np.einsum("ab,nbc->nac", D, base["out"])
        rms = np.sqrt(np.mean(base["out"] ** 2))
        assert np.max(np.abs(o["out"] - want)) / rms < 1e-10


def test_target_subset_matches_full():
    wl = W.make_workload("c1")
    full = layer.layer_forward_workload(wl)
    sub = np.array([0, 17, 100, 255])
    part = layer.layer_forward_workload(wl, targets=sub)
    assert np.max(np.abs(part["out"] - full["out"][sub])) < 1e-13


# ---------------------------------------------------------------- envelope beyond the cutoff
def test_envelope_is_zero_from_the_cutoff_on():
    """The cosine envelope is the cutoff mask of the FlashSchNet page (section 2.2):
    f_c(d) = 0 for d >= r_c.  (cos(pi d / r_c) + 1) / 2 itself would rise again
    beyond r_c (0.0089 at 5.3 A for r_c = 5) and return to 1 at 2 r_c."""
    rc, R = 5.0, 8
    w = RNG.standard_normal((R, 3))
    d = np.array([5.0, 5.0 + 1e-9, 5.3, 5.5, 7.5, 10.0, 12.0])
    assert np.all(layer.rbf_bias(d, w, rc) == 0.0)
    below = layer.rbf_bias(np.array([5.0 - 1e-3]), np.ones((R, 1)), rc)[0, 0]
    assert 0.0 < below < 1e-6                        # continuous at r_c from below
    # the torch form (gradients) agrees: value and slope 0 beyond r_c
    from oracle import backward
    dt = torch.tensor([4.0, 5.3, 6.0], dtype=torch.float64, requires_grad=True)
    b = backward.rbf_bias_torch(dt, w, rc)
    assert np.all(b[1:].detach().numpy() == 0.0)
    b.sum().backward()
    assert dt.grad[0] != 0.0 and np.all(dt.grad[1:].numpy() == 0.0)


def test_listed_pair_beyond_cutoff_gets_no_bias():
    """Reused list (Tessera article, neighbour reuse): target 0 lists atom 1 at
    3 A and atom 2 at 5.4 A, past r_c = 5.  With W_Q = W_K = 0 the logits are the
    biases alone: b(3 A) from the Gaussians and the envelope written out here, and 0
    for the pair beyond r_c, so alpha = (e^b, 1) / (e^b + 1) per head."""
    C, H, R, L, rc = 8, 2, 6, 2, 5.0
    p = _rand_layer(3, C, H, R, L, 1.0, 31)
    p["pos"] = np.array([[0.2, -0.1, 0.3], [0.2, -0.1, 3.3], [5.6, -0.1, 0.3]])
    p["w_q"] = np.zeros((C, C))
    p["w_k"] = np.zeros((C, C))
    rows = [np.array([1, 2], dtype=np.int32), np.array([0], dtype=np.int32), np.array([0], dtype=np.int32)]
    o = layer.layer_forward(**p, lmax=L, heads=H, cutoff=rc, rows=rows)
    delta = rc / (R - 1)
    d = 3.0
    fc = 0.5 * (math.cos(math.pi * d / rc) + 1.0)
    b = np.array([fc * sum(p["w_rbf"][k, h] * math.exp(-((d - k * delta) ** 2) / (2 * delta * delta))
                           for k in range(R)) for h in range(H)])
    a1 = np.exp(b) / (np.exp(b) + 1.0)                 # per head
    head_of = np.arange(C) // (C // H)
    hp = {int(s): o["hprime"][t] for t, s in enumerate(o["src"])}
    want = a1[head_of] * hp[1] + (1.0 - a1[head_of]) * hp[2]
    assert np.max(np.abs(o["m"][0] - want)) < 1e-13
    # with the unclamped envelope the far pair would carry f_c(5.4 A) = 0.0157 of its sum
    assert abs(0.5 * (math.cos(math.pi * 5.4 / rc) + 1.0) - 0.0157) < 1e-4


# ---------------------------------------------------------------- per-degree weights
def test_per_degree_value_and_output_weights():
    """W_V[l] acts on degree l of the input and W_O[l] on degree l of the output
    (readings R12, R14).  One neighbour (alpha = 1), input nonzero in degree l_i only,
    W_V[l] = s_l I and W_O[l] = t_l I with distinct s_l, t_l: block l_o of the output
    is s_{l_i} t_{l_o} times the output with identity weights.  Taking W_V[0] for
    every degree, or W_O of a neighbouring degree, breaks the factor."""
    C, H, L, rc = 8, 2, 3, 4.0
    p = _rand_layer(2, C, H, 5, L, 1.0, 41)
    p["pos"] = np.array([[0.3, -0.7, 1.1], [-1.2, 0.4, 2.0]])
    rows = [np.array([1], dtype=np.int32), np.array([0], dtype=np.int32)]
    s = np.array([0.5, 2.0, -3.0, 7.0])
    t = np.array([11.0, -0.25, 4.0, 0.125])
    eye = np.broadcast_to(np.eye(C), (L + 1, C, C))
    sl = so3.block_slices(L)
    for li in range(L + 1):
        h = np.zeros_like(p["h"])
        h[:, sl[li], :] = p["h"][:, sl[li], :]
        base = dict(p, h=h, w_v=eye.copy(), w_o=eye.copy())
        ref = layer.layer_forward(**base, lmax=L, heads=H, cutoff=rc, rows=rows)["out"]
        scaled = dict(base, w_v=s[:, None, None] * eye, w_o=t[:, None, None] * eye)
        out = layer.layer_forward(**scaled, lmax=L, heads=H, cutoff=rc, rows=rows)["out"]
        nonzero = 0
        for lo in range(L + 1):
            want = s[li] * t[lo] * ref[:, sl[lo], :]
            assert np.max(np.abs(out[:, sl[lo], :] - want)) <= 1e-13 * max(1.0, np.max(np.abs(want)))
            nonzero += np.max(np.abs(want)) > 1e-6
        assert nonzero >= 2                                # several output degrees are fed
