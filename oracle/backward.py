"""fp64 oracle of one layer's gradient with respect to its input features h.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product path never does.

B1  L(h) = sum(g * out(h)) for a fixed upstream gradient g; the oracle returns
    dL/dh.  The layer of layer.py (O4-O8) is written again with torch fp64
    operations -- projections, dense Clebsch-Gordan tensor products with the real
    spherical harmonics of each position (held constant: so3.coupling_tensor,
    so3.real_sh), the distance bias (constant: layer.rbf_bias), an explicit
    per-head softmax over each neighbour set -- and reverse-mode differentiation
    gives the gradient.  Positions, weights and neighbour lists are fixed.
    The forward pass here is checked against layer.layer_forward, and the
    gradient against central finite differences of layer.layer_forward.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import layer, so3

__all__ = ["layer_forward_torch", "grad_h"]


def _tp(x, Y, w, lmax: int):
    """out^{l_o}[n, m_o, c] = sum_p w[p, c] sum T_p[m_i, m_f, m_o] x^{l_i}[n, m_i, c] Y^{l_f}[n, m_f]."""
    sl = so3.block_slices(lmax)
    blocks = [None] * (lmax + 1)
    for p, (li, lf, lo) in enumerate(so3.paths(lmax)):
        T = torch.from_numpy(np.array(so3.coupling_tensor(li, lf, lo)))
        term = torch.einsum("ijk,nic,nj->nkc", T, x[:, sl[li], :], Y[:, sl[lf]]) * w[p][None, None, :]
        blocks[lo] = term if blocks[lo] is None else blocks[lo] + term
    return torch.cat(blocks, dim=1)


def layer_forward_torch(pos, h, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt, *, lmax: int, heads: int,
                        cutoff: float, rows, targets=None):
    """The layer in torch fp64 for ``targets`` (default every atom; rows[t] is the
    row of targets[t]); h [n, (L+1)^2, C] may require grad."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    pos = np.asarray(pos, dtype=np.float64)
    cutoff = float(np.float32(cutoff))
    n, nc, C = h.shape
    tg = np.arange(n) if targets is None else np.asarray(targets, dtype=np.int64)
    d_head = C // heads
    head_of = torch.arange(C) // d_head
    sl = so3.block_slices(lmax)
    q = h[:, 0, :] @ t(w_q)
    k = h[:, 0, :] @ t(w_k)
    v = torch.cat([h[:, sl[l], :] @ t(w_v[l]) for l in range(lmax + 1)], dim=1)
    Y = t(so3.real_sh(pos, lmax))
    hp = _tp(v, Y, t(w_src), lmax)
    ms = []
    for ti, i in enumerate(tg):
        js = np.asarray(rows[ti], dtype=np.int64)
        if js.size == 0:
            ms.append(torch.zeros(nc, C, dtype=torch.float64))
            continue
        diff = pos[js] - pos[i][None, :]
        d = np.sqrt(np.sum(diff * diff, axis=1))
        bias = t(layer.rbf_bias(d, w_rbf, cutoff))                           # [J, H]
        jt = torch.from_numpy(js)
        qk = (k[jt] * q[i][None, :]).reshape(js.size, heads, d_head).sum(dim=2)
        alpha = torch.softmax(qk / math.sqrt(d_head) + bias, dim=0)          # [J, H]
        ms.append(torch.einsum("jc,jkc->kc", alpha[:, head_of], hp[jt]))
    m = torch.stack(ms, dim=0)
    hhat = _tp(m, Y[torch.from_numpy(tg)], t(w_tgt), lmax)
    return torch.cat([hhat[:, sl[l], :] @ t(w_o[l]) for l in range(lmax + 1)], dim=1)


def grad_h(pos, h, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt, g, *, lmax: int, heads: int, cutoff: float, rows,
           targets=None):
    """dL/dh for L = sum over ``targets`` (default all) of g[t] * out[t]; g has one
    row per target.

    B2  Sampling: out_i depends on h_i and on h_j for j in row i only, so for a
    symmetric list the gradient at atom a is exact when the targets cover a and
    every member of row a."""
    ht = torch.tensor(np.asarray(h, dtype=np.float64), requires_grad=True)
    out = layer_forward_torch(pos, ht, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt, lmax=lmax, heads=heads,
                              cutoff=cutoff, rows=rows, targets=targets)
    (out * torch.as_tensor(np.asarray(g, dtype=np.float64))).sum().backward()
    return ht.grad.numpy()
