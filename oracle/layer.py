"""fp64 oracle of one E2Former-V2 node-centric equivariant attention layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product path never does.

The layer, step by step (O1..O8), each written as its plain definition:

O1 neighbours  -- brute force over all pairs with the fp64 predicate of
                  brute_neighbors.c against the square of the cutoff's fp32
                  value; with a cap K, keep the K nearest by (d^2, j); rows
                  sorted by j.  (Explainer section 5.2: verify
                  the neighbour list; section 3.2: K = 256 with masked padding.)
O2 encoding    -- real spherical harmonics of the unit position vector
                  (so3.real_sh; explainer section 2.3).
O3 coupling    -- real Clebsch-Gordan tensors (so3.coupling_tensor).
O4 projections -- q = h^0 W_Q, k = h^0 W_K (the l = 0 block, so attention
                  weights are invariant: direction enters only through the
                  value path, explainer section 3.1); v^l = h^l W_V[l].
O5 source TP   -- h'_j = sum_p w_src[p] (v_j (x) Y(r_j))_p, full dense CG sum,
                  no EAAS (explainer section 3.1, source pre-coupling).
O6 attention   -- b_h(d) = f_c(d) sum_k W_rbf[k, h] phi_k(d), Gaussian RBFs
                  phi_k(d) = exp(-(d - mu_k)^2 / (2 Delta^2)), mu_k = k r_c/(R-1),
                  Delta = r_c/(R-1), cosine envelope f_c(d) = (cos(pi d / r_c) + 1)/2
                  for d < r_c and 0 from r_c on (FlashSchNet page, section 2.1:
                  distance, Gaussian expansion and cosine envelope; section 2.2:
                  the cutoff mask.  A listed pair beyond r_c -- a reused list after
                  the atoms moved, Tessera article, neighbour reuse -- gets no bias,
                  while its q.k term still counts);
                  s_jh = q_i^h . k_j^h / sqrt(C/H) + b_h(d_ij);
                  alpha = explicit softmax over the whole neighbour set;
                  m_i[l, m, c] = sum_j alpha_{j, head(c)} h'_j[l, m, c]
                  (explainer section 3.1 streaming aggregation; section 3.2 says the
                  online softmax with running max and normaliser computes exactly
                  this).  An empty set gives m_i = 0.
O7 target TP   -- hhat_i = sum_p w_tgt[p] (m_i (x) Y(r_i))_p (explainer section 3.1).
O8 output      -- out_i^l = hhat_i^l W_O[l].

Head h owns channels [h*d, (h+1)*d), d = C/H, in every (l, m) component.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

from . import so3

__all__ = ["neighbors", "neighbors_numpy", "rbf_bias", "project", "source_coupling",
           "attention", "layer_forward", "build_c", "rows_to_csr"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "brute_neighbors.c")
_LIB = os.path.join(_HERE, "liboracle_nbr.so")
_lib = None


def build_c(force: bool = True) -> str:
    """Compile the brute-force neighbour search (plain C, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        "-shared", "-fPIC", "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_c(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_nbr_count.restype = ctypes.c_int64
        lib.oracle_nbr_count.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
        lib.oracle_nbr_fill.restype = None
        lib.oracle_nbr_fill.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def _cap_and_sort(idx: np.ndarray, d2: np.ndarray, k: int) -> np.ndarray:
    if k > 0 and idx.size > k:
        order = np.lexsort((idx, d2))[:k]     # primary d2, then j
        idx = idx[order]
    return np.sort(idx).astype(np.int32)


def neighbors(pos: np.ndarray, cutoff: float, max_neighbors: int = 0, targets=None):
    """Neighbour rows for ``targets`` (default all): a list of int32 arrays sorted by j."""
    pos32 = np.ascontiguousarray(np.asarray(pos, dtype=np.float64).astype(np.float32))
    n = pos32.shape[0]
    tg = np.arange(n, dtype=np.int32) if targets is None else np.ascontiguousarray(targets, dtype=np.int32)
    rc = float(np.float32(cutoff))          # the cutoff is given as an fp32 value
    rc2 = rc * rc
    lib = _load()
    counts = np.zeros(tg.size, dtype=np.int64)
    total = lib.oracle_nbr_count(pos32.ctypes.data, n, tg.ctypes.data, tg.size, rc2, counts.ctypes.data)
    offs = np.zeros(tg.size + 1, dtype=np.int64)
    np.cumsum(counts, out=offs[1:])
    idx = np.zeros(max(total, 1), dtype=np.int32)
    d2 = np.zeros(max(total, 1), dtype=np.float64)
    lib.oracle_nbr_fill(pos32.ctypes.data, n, tg.ctypes.data, tg.size, rc2, offs.ctypes.data,
                        idx.ctypes.data, d2.ctypes.data)
    return [_cap_and_sort(idx[offs[t]:offs[t + 1]], d2[offs[t]:offs[t + 1]], max_neighbors)
            for t in range(tg.size)]


def neighbors_numpy(pos: np.ndarray, cutoff: float, max_neighbors: int = 0, targets=None):
    """Same definition in numpy (slow path; used to cross-check the C search)."""
    p = np.asarray(pos, dtype=np.float64).astype(np.float32).astype(np.float64)
    n = p.shape[0]
    tg = np.arange(n) if targets is None else np.asarray(targets)
    rc = float(np.float32(cutoff))
    rc2 = rc * rc
    rows = []
    for i in tg:
        dx = p[:, 0] - p[i, 0]
        dy = p[:, 1] - p[i, 1]
        dz = p[:, 2] - p[i, 2]
        d2 = (dx * dx + dy * dy) + dz * dz
        mask = d2 < rc2
        mask[i] = False
        j = np.nonzero(mask)[0]
        rows.append(_cap_and_sort(j, d2[j], max_neighbors))
    return rows


def rows_to_csr(rows):
    lens = np.array([r.size for r in rows], dtype=np.int64)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    idx = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, dtype=np.int32)
    return start, lens, idx


def rbf_bias(d: np.ndarray, w_rbf: np.ndarray, cutoff: float) -> np.ndarray:
    """b[..., h] = f_c(d) * sum_k W_rbf[k, h] exp(-(d - mu_k)^2 / (2 Delta^2)),
    f_c(d) = (cos(pi d / r_c) + 1) / 2 below r_c and 0 from r_c on (the cutoff mask)."""
    d = np.asarray(d, dtype=np.float64)
    R = w_rbf.shape[0]
    delta = cutoff / (R - 1)
    mu = np.arange(R, dtype=np.float64) * delta
    phi = np.exp(-((d[..., None] - mu) ** 2) / (2.0 * delta * delta))
    fc = np.where(d < cutoff, 0.5 * (np.cos(np.pi * d / cutoff) + 1.0), 0.0)
    return fc[..., None] * (phi @ np.asarray(w_rbf, dtype=np.float64))


def project(h: np.ndarray, w_q, w_k, w_v, lmax: int):
    """O4: q, k from the l = 0 block; v^l = h^l W_V[l]."""
    h = np.asarray(h, dtype=np.float64)
    q = h[:, 0, :] @ w_q
    k = h[:, 0, :] @ w_k
    v = np.empty_like(h)
    for l, sl in enumerate(so3.block_slices(lmax)):
        v[:, sl, :] = h[:, sl, :] @ w_v[l]
    return q, k, v


def source_coupling(v: np.ndarray, pos: np.ndarray, w_src: np.ndarray, lmax: int) -> np.ndarray:
    """O5: h' = full-CG tensor product of v with Y(r) (no EAAS)."""
    return so3.tensor_product(v, pos, w_src, lmax)


def attention(q_i, pos_i, rows, k, hp, pos, w_rbf, cutoff: float, heads: int):
    """O6 for a batch of targets: explicit softmax over each neighbour set.

    q_i: [T, C]; pos_i: [T, 3]; rows: list of T index arrays into k / hp / pos.
    Returns m [T, n_comp, C].
    """
    T = len(rows)
    C = k.shape[1]
    d_head = C // heads
    head_of = np.arange(C) // d_head
    m = np.zeros((T,) + hp.shape[1:])
    for t, js in enumerate(rows):
        if js.size == 0:
            continue
        diff = pos[js] - pos_i[t][None, :]
        d = np.sqrt(np.sum(diff * diff, axis=1))
        bias = rbf_bias(d, w_rbf, cutoff)                            # [J, H]
        qk = (k[js] * q_i[t][None, :]).reshape(js.size, heads, d_head).sum(axis=2)
        s = qk / math.sqrt(d_head) + bias                            # [J, H]
        e = np.exp(s - s.max(axis=0, keepdims=True))
        alpha = e / e.sum(axis=0, keepdims=True)                     # [J, H]
        m[t] = np.einsum("jc,jkc->kc", alpha[:, head_of], hp[js])
    return m


def layer_forward(pos, h, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt, *, lmax: int, heads: int,
                  cutoff: float, max_neighbors: int = 0, targets=None, rows=None):
    """Whole layer for ``targets`` (default all atoms), all intermediates in fp64.

    Only the sources the targets need are coupled, so a small target sample of a
    large system is cheap.  Returns a dict with rows, q, k, v, hprime (indexed by
    atom id through ``src``), m, hhat and out for the targets.
    """
    pos = np.asarray(pos, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    cutoff = float(np.float32(cutoff))       # the cutoff is given as an fp32 value
    n = pos.shape[0]
    tg = np.arange(n) if targets is None else np.asarray(targets, dtype=np.int64)
    if rows is None:
        rows = neighbors(pos, cutoff, max_neighbors, targets=tg)
    src = np.unique(np.concatenate([np.asarray(r, dtype=np.int64) for r in rows] + [np.zeros(0, np.int64)]))
    # O4 on the atoms needed: targets (q) and sources (k, v)
    q_t, _, _ = project(h[tg], w_q, w_k, w_v, lmax)
    _, k_s, v_s = project(h[src], w_q, w_k, w_v, lmax)
    # O5 on the sources
    hp_s = source_coupling(v_s, pos[src], w_src, lmax)
    # Re-index rows into the compact source arrays
    where = np.full(n, -1, dtype=np.int64)
    where[src] = np.arange(src.size)
    rows_c = [where[np.asarray(r, dtype=np.int64)] for r in rows]
    # O6
    m = attention(q_t, pos[tg], rows_c, k_s, hp_s, pos[src], w_rbf, cutoff, heads)
    # O7
    hhat = so3.tensor_product(m, pos[tg], w_tgt, lmax)
    # O8
    out = np.empty_like(hhat)
    for l, sl in enumerate(so3.block_slices(lmax)):
        out[:, sl, :] = hhat[:, sl, :] @ w_o[l]
    return {"targets": tg, "rows": rows, "src": src, "q": q_t, "k": k_s, "v": v_s,
            "hprime": hp_s, "m": m, "hhat": hhat, "out": out}


def layer_forward_workload(wl, targets=None, rows=None):
    """Convenience wrapper taking a workloads.Workload-like object (duck typed)."""
    c = wl.cfg
    return layer_forward(wl.pos, wl.h, wl.w_q, wl.w_k, wl.w_v, wl.w_o, wl.w_rbf, wl.w_src, wl.w_tgt,
                         lmax=c.lmax, heads=c.heads, cutoff=c.cutoff, max_neighbors=c.max_neighbors,
                         targets=targets, rows=rows)
