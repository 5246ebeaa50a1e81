"""fp64 oracle of one layer's gradient with respect to its input features h.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product path never does.

B1  L(h) = sum(g * out(h)) for a fixed upstream gradient g; the oracle returns
    dL/dh.  The layer of layer.py (O4-O8) is written again with torch fp64
    operations -- projections, dense Clebsch-Gordan tensor products with the real
    spherical harmonics of each position (held constant: so3.coupling_tensor,
    so3.real_sh), the distance bias (constant: layer.rbf_bias), an explicit
    per-head softmax over each neighbour set -- and reverse-mode differentiation
    gives the gradient.  Weights and neighbour lists are fixed.
    The forward pass here is checked against layer.layer_forward, and the
    gradient against central finite differences of layer.layer_forward.

B3  L(pos, h) as in B1 with the positions free as well: dL/dpos through the
    encodings Y(r_i) of both couplings and through every pair distance in the
    bias, with the neighbour lists held fixed.  The envelope and its slope are 0
    from the cutoff on (layer.rbf_bias), so a listed pair beyond it -- a reused
    list after the atoms moved -- adds no bias term to dL/dpos, and a pair
    crossing the cutoff sees no jump in either.  At a
    zero position vector the direction is undefined: its encoding is held
    constant, so that atom's position receives only the bias terms.

B4  A stack of layers (each the B3 function of the previous output) with the
    lists held fixed; for bf16 storage the outputs between layers are rounded to
    bf16 as stack.stack_step does and the rounding passes the gradient through
    unchanged (a step function has no useful derivative; this is the reading the
    GPU stack gradient follows).  Pinned against the chain rule written out with
    separate per-layer gradients.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import layer, so3, stack

__all__ = ["layer_forward_torch", "grad_h", "grad_pos_h", "stack_grad_pos_h", "real_sh_torch", "rbf_bias_torch"]


def real_sh_torch(r, lmax: int):
    """so3.real_sh in torch (differentiable in r): the same closed forms of the
    direction r / |r|; a zero vector maps to Y_0 = 1, Y_{l>0} = 0, held constant
    (the direction, and so its derivative, is not defined there: B3)."""
    n2 = torch.sum(r * r, dim=-1)
    zero = n2 == 0.0
    safe = torch.sqrt(torch.where(zero, torch.ones_like(n2), n2))     # no sqrt at 0: its slope is infinite
    u = r / safe[..., None]
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    out = [torch.ones_like(x)]
    if lmax >= 1:
        s3 = math.sqrt(3.0)
        out += [s3 * y, s3 * z, s3 * x]
    if lmax >= 2:
        s15, s5 = math.sqrt(15.0), math.sqrt(5.0)
        out += [s15 * x * y, s15 * y * z, 0.5 * s5 * (3.0 * z * z - 1.0), s15 * x * z, 0.5 * s15 * (x * x - y * y)]
    if lmax >= 3:
        a, b, c = math.sqrt(35.0 / 8.0), math.sqrt(105.0), math.sqrt(21.0 / 8.0)
        out += [a * y * (3 * x * x - y * y), b * x * y * z, c * y * (5 * z * z - 1),
                0.5 * math.sqrt(7.0) * (5 * z ** 3 - 3 * z), c * x * (5 * z * z - 1),
                0.5 * b * z * (x * x - y * y), a * x * (x * x - 3 * y * y)]
    Y = torch.stack(out, dim=-1)
    keep = torch.ones_like(Y)
    keep[..., 1:] = (~zero).to(Y.dtype)[..., None]
    return Y * keep


def rbf_bias_torch(d, w_rbf, cutoff: float):
    """layer.rbf_bias in torch (differentiable in d; value and slope 0 from the cutoff on)."""
    w = torch.as_tensor(np.asarray(w_rbf, dtype=np.float64))
    R = w.shape[0]
    delta = cutoff / (R - 1)
    mu = torch.arange(R, dtype=torch.float64) * delta
    phi = torch.exp(-((d[..., None] - mu) ** 2) / (2.0 * delta * delta))
    fc = torch.where(d < cutoff, 0.5 * (torch.cos(math.pi * d / cutoff) + 1.0), torch.zeros_like(d))
    return fc[..., None] * (phi @ w)


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
    row of targets[t]); h [n, (L+1)^2, C] may require grad, and so may pos when it
    is given as a torch tensor (then the encodings and the distance bias follow it)."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    pos_t = pos if torch.is_tensor(pos) else torch.as_tensor(np.asarray(pos, dtype=np.float64))
    cutoff = float(np.float32(cutoff))
    n, nc, C = h.shape
    tg = np.arange(n) if targets is None else np.asarray(targets, dtype=np.int64)
    d_head = C // heads
    head_of = torch.arange(C) // d_head
    sl = so3.block_slices(lmax)
    q = h[:, 0, :] @ t(w_q)
    k = h[:, 0, :] @ t(w_k)
    v = torch.cat([h[:, sl[l], :] @ t(w_v[l]) for l in range(lmax + 1)], dim=1)
    Y = real_sh_torch(pos_t, lmax)
    hp = _tp(v, Y, t(w_src), lmax)
    ms = []
    for ti, i in enumerate(tg):
        js = np.asarray(rows[ti], dtype=np.int64)
        if js.size == 0:
            ms.append(torch.zeros(nc, C, dtype=torch.float64))
            continue
        jt = torch.from_numpy(js)
        diff = pos_t[jt] - pos_t[int(i)][None, :]
        d = torch.sqrt(torch.sum(diff * diff, dim=1))
        bias = rbf_bias_torch(d, w_rbf, cutoff)                              # [J, H]
        qk = (k[jt] * q[i][None, :]).reshape(js.size, heads, d_head).sum(dim=2)
        alpha = torch.softmax(qk / math.sqrt(d_head) + bias, dim=0)          # [J, H]
        ms.append(torch.einsum("jc,jkc->kc", alpha[:, head_of], hp[jt]))
    m = torch.stack(ms, dim=0)
    hhat = _tp(m, Y[torch.from_numpy(tg)], t(w_tgt), lmax)
    return torch.cat([hhat[:, sl[l], :] @ t(w_o[l]) for l in range(lmax + 1)], dim=1)


def grad_pos_h(pos, h, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt, g, *, lmax: int, heads: int, cutoff: float,
               rows, targets=None):
    """(dL/dpos, dL/dh) for L = sum over ``targets`` of g[t] * out[t] (B3)."""
    pt = torch.tensor(np.asarray(pos, dtype=np.float64), requires_grad=True)
    ht = torch.tensor(np.asarray(h, dtype=np.float64), requires_grad=True)
    out = layer_forward_torch(pt, ht, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt, lmax=lmax, heads=heads,
                              cutoff=cutoff, rows=rows, targets=targets)
    (out * torch.as_tensor(np.asarray(g, dtype=np.float64))).sum().backward()
    return pt.grad.numpy(), ht.grad.numpy()


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


def stack_grad_pos_h(pos, h0, layers, rows_by_cutoff, g, round_between: bool = False):
    """B4: (dL/dpos, dL/dh0) for L = sum(g * out) of a layer stack: layer l + 1 takes
    layer l's output (the composition of stack.stack_step), each layer on the rows
    of its cutoff, the lists held fixed.  ``layers``: Workload-like weight sets with
    a cfg (lmax, heads, cutoff); ``rows_by_cutoff``: {fp32 cutoff: rows}.
    round_between = False: the real-valued composition, no rounding between layers.
    round_between = True (bf16 storage): each non-final output is rounded to bf16
    before it feeds the next layer, as in stack.stack_step, and the rounding passes
    the gradient through unchanged (its derivative taken as the identity), so every
    layer is differentiated at the input it actually receives."""
    pt = torch.tensor(np.asarray(pos, dtype=np.float64), requires_grad=True)
    ht = torch.tensor(np.asarray(h0, dtype=np.float64), requires_grad=True)
    x = ht
    for li, wl in enumerate(layers):
        c = wl.cfg
        rows = rows_by_cutoff[float(np.float32(c.cutoff))]
        if round_between and li > 0:
            xr = torch.as_tensor(stack._round_bf16(x.detach().numpy()))
            x = x + (xr - x).detach()
        x = layer_forward_torch(pt, x, wl.w_q, wl.w_k, wl.w_v, wl.w_o, wl.w_rbf, wl.w_src, wl.w_tgt, lmax=c.lmax,
                                heads=c.heads, cutoff=c.cutoff, rows=rows)
    (x * torch.as_tensor(np.asarray(g, dtype=np.float64))).sum().backward()
    return pt.grad.numpy(), ht.grad.numpy()
