"""fp64 oracle of the exact edge-equivalent form of the attention layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product path never does.

The E2Former-V2 explainer (section 1.2) names the Wigner-6j recoupling identity
as the mathematics that lets a node-centric evaluation reproduce an
edge-centric one.  What is reproduced is a tensor product on every edge with
the geometric encoding of the edge vector; for the node-centric split to be
exact the encoding must be a polynomial in the edge vector, i.e. the solid
harmonics.  This module writes that edge form out as its plain definition,
edge by edge, with no recoupling:

E1 encoding     -- S^l(x) = |x|^l Y^l(x / |x|), the component-normalised real
                  solid harmonic (a homogeneous polynomial of degree l; S^0 = 1,
                  and S^{l>0}(0) = 0), of the edge vector scaled by the cutoff,
                  x_ij = (r_j - r_i) / r_c.
E2 edge product -- e_ij = sum_p w_e[p, c] (v_j (x) S(x_ij))_p over every path
                  p = (l_i, l_f, l_o) of so3.paths, full dense Clebsch-Gordan
                  sum (so3.coupling_tensor), one weight per path and channel;
                  v = the per-degree value projection of layer.project (O4).
E3 attention    -- the layer's weights alpha_ij (O6: q.k / sqrt(d) plus the
                  Gaussian-RBF x cosine-cutoff bias, explicit softmax over the
                  neighbour set); m_i = sum_j alpha_ij e_ij (0 for an empty set).
E4 output       -- out_i^l = m_i^l W_O[l].

Because S depends on r_j - r_i only, the result is invariant under a common
translation of all positions, which the node-centric layer (encodings of the
positions themselves) is not.
"""
from __future__ import annotations

import math

import numpy as np

from . import layer, so3

__all__ = ["solid_sh", "edge_product", "edge_forward"]


def solid_sh(x: np.ndarray, lmax: int) -> np.ndarray:
    """S^l(x) = |x|^l Y^l(x / |x|) for l <= lmax, [..., (lmax+1)^2]; S(0) = (1, 0, ...)."""
    x = np.asarray(x, dtype=np.float64)
    Y = so3.real_sh(x, lmax)
    r = np.linalg.norm(x, axis=-1)
    out = Y.copy()
    for l, sl in enumerate(so3.block_slices(lmax)):
        out[..., sl] *= (r ** l)[..., None]
    return out


def edge_product(v: np.ndarray, S: np.ndarray, w: np.ndarray, lmax: int) -> np.ndarray:
    """E2 for a batch of edges: v [E, (L+1)^2, C], S [E, (L+1)^2] -> [E, (L+1)^2, C]."""
    sl = so3.block_slices(lmax)
    out = np.zeros_like(v)
    for p, (li, lf, lo) in enumerate(so3.paths(lmax)):
        T = so3.coupling_tensor(li, lf, lo)
        term = np.einsum("ijk,eic,ej->ekc", T, v[:, sl[li], :], S[:, sl[lf]], optimize=True)
        out[:, sl[lo], :] += term * w[p][None, None, :]
    return out


def edge_forward(pos, h, w_q, w_k, w_v, w_o, w_rbf, w_edge, *, lmax: int, heads: int, cutoff: float, rows,
                 targets=None):
    """E1-E4 for ``targets`` (default every atom; rows[t] is the row of targets[t]).
    Returns a dict with m (the aggregated edge products) and out, both fp64."""
    pos = np.asarray(pos, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    cutoff = float(np.float32(cutoff))              # the cutoff is given as an fp32 value
    n = pos.shape[0]
    tg = np.arange(n) if targets is None else np.asarray(targets, dtype=np.int64)
    q, k, v = layer.project(h, w_q, w_k, w_v, lmax)
    C = h.shape[2]
    d_head = C // heads
    head_of = np.arange(C) // d_head
    m = np.zeros((tg.size,) + h.shape[1:])
    for t, i in enumerate(tg):
        js = np.asarray(rows[t], dtype=np.int64)
        js = js[(js >= 0) & (js < n)]
        if js.size == 0:
            continue
        diff = pos[js] - pos[i][None, :]
        d = np.sqrt(np.sum(diff * diff, axis=1))
        s = (k[js] * q[i][None, :]).reshape(js.size, heads, d_head).sum(axis=2) / math.sqrt(d_head)
        s = s + layer.rbf_bias(d, w_rbf, cutoff)
        e = np.exp(s - s.max(axis=0, keepdims=True))
        alpha = e / e.sum(axis=0, keepdims=True)                                  # [J, H]
        edges = edge_product(v[js], solid_sh(diff / cutoff, lmax), np.asarray(w_edge, dtype=np.float64), lmax)
        m[t] = np.einsum("jc,jkc->kc", alpha[:, head_of], edges)
    out = np.empty_like(m)
    for l, sl in enumerate(so3.block_slices(lmax)):
        out[:, sl, :] = m[:, sl, :] @ w_o[l]
    return {"targets": tg, "m": m, "out": out}
