"""fp64 oracle of a stack of node-centric attention layers over a moving system.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product path never does.

What is computed (Tessera article, the model description and the neighbour
reuse paragraph), step by step:

S1 layers      -- three short-range layers (5 A) and one long-range layer (8 A),
                  applied in the order given; layer l + 1 takes layer l's output
                  as its input features (the pages give no residual or norm
                  between layers; the plain composition is taken).  In 16-bit
                  storage a layer's input is stored in bf16, so the output is
                  rounded to bf16 (nearest even) before it feeds the next layer.
S2 topology    -- the neighbour topology is reused between rebuilds while every
                  layer takes distances (and directions) from the current
                  positions.  A rebuild builds the list at the largest cutoff
                  (K nearest when capped, layer.neighbors) and, for each smaller
                  cutoff, keeps the entries of that list within it, both decided
                  at the rebuild positions with the fp64 predicate of the
                  neighbour search.
S3 rebuild     -- a rebuild happens at the first step, when `rebuild_every`
                  steps have passed since the last one, and earlier when some
                  atom lies more than `max_disp` from its position at the last
                  rebuild: d2 = (dx*dx + dy*dy) + dz*dz in fp64 with
                  dx = x - x_ref (fp32 values, so dx is exact), compared with
                  max_disp^2 (max_disp's fp32 value, squared in fp64).
                  A non-finite d2 also triggers a rebuild.
"""
from __future__ import annotations

import numpy as np

from . import layer

__all__ = ["filter_rows", "max_displacement2", "stack_step", "StackState", "run_stack"]


def _d2(p: np.ndarray, i: int, js: np.ndarray) -> np.ndarray:
    """The neighbour search's fp64 squared distance, each operation rounded."""
    dx = p[js, 0] - p[i, 0]
    dy = p[js, 1] - p[i, 1]
    dz = p[js, 2] - p[i, 2]
    return (dx * dx + dy * dy) + dz * dz


def filter_rows(pos: np.ndarray, rows, cutoff: float):
    """S2: the entries of each row within ``cutoff`` (its fp32 value), order kept."""
    p = np.asarray(pos, dtype=np.float64).astype(np.float32).astype(np.float64)
    rc = float(np.float32(cutoff))
    rc2 = rc * rc
    out = []
    for i, r in enumerate(rows):
        r = np.asarray(r, dtype=np.int64)
        r = r[(r >= 0) & (r < p.shape[0])]
        out.append(r[_d2(p, i, r) < rc2].astype(np.int32) if r.size else r.astype(np.int32))
    return out


def max_displacement2(pos: np.ndarray, ref: np.ndarray) -> float:
    """S3: the largest squared displacement, fp64, non-finite values as +inf."""
    p = np.asarray(pos, dtype=np.float64).astype(np.float32).astype(np.float64)
    q = np.asarray(ref, dtype=np.float64).astype(np.float32).astype(np.float64)
    dx, dy, dz = p[:, 0] - q[:, 0], p[:, 1] - q[:, 1], p[:, 2] - q[:, 2]
    d2 = (dx * dx + dy * dy) + dz * dz
    d2 = np.where(np.isfinite(d2), d2, np.inf)
    return float(d2.max()) if d2.size else 0.0


class StackState:
    """What persists between steps: reference positions, the lists per cutoff,
    steps since the last rebuild."""

    def __init__(self, cutoffs, max_neighbors: int, rebuild_every: int = 10, max_disp: float = 0.25):
        self.cutoffs = [float(np.float32(c)) for c in cutoffs]
        self.K = int(max_neighbors)
        self.rebuild_every = int(rebuild_every)
        self.max_disp = float(np.float32(max_disp))
        self.ref = None
        self.rows = {}
        self.since = -1
        self.rebuilds = []

    def need_rebuild(self, pos) -> bool:
        if self.since < 0 or self.since >= self.rebuild_every:
            return True
        return not (max_displacement2(pos, self.ref) <= self.max_disp * self.max_disp)

    def rebuild(self, pos, step: int):
        top = max(self.cutoffs)
        rows = layer.neighbors(pos, top, self.K)
        self.rows = {top: rows}
        for c in sorted(set(self.cutoffs)):
            if c != top:
                self.rows[c] = filter_rows(pos, rows, c)
        self.ref = np.asarray(pos, dtype=np.float64).copy()
        self.since = 0
        self.rebuilds.append(step)


def stack_step(state: StackState, pos, h0, layers, step: int, storage: str):
    """One model step: S3 (rebuild if due), then S1 over the lists of S2.
    ``layers`` are Workload-like weight sets (duck typed: w_q ... w_tgt and a cfg
    with lmax, heads, cutoff).  Returns the last layer's output."""
    if state.need_rebuild(pos):
        state.rebuild(pos, step)
    h = np.asarray(h0, dtype=np.float64)
    out = None
    for li, wl in enumerate(layers):
        c = wl.cfg
        rows = state.rows[float(np.float32(c.cutoff))]
        r = layer.layer_forward(pos, h, wl.w_q, wl.w_k, wl.w_v, wl.w_o, wl.w_rbf, wl.w_src, wl.w_tgt,
                                lmax=c.lmax, heads=c.heads, cutoff=c.cutoff, rows=rows)
        out = r["out"]
        if li + 1 < len(layers):         # the next layer's input in the storage dtype ("fp64": kept)
            if storage == "bf16":
                h = _round_bf16(out)
            elif storage == "fp32":
                h = out.astype(np.float32).astype(np.float64)
            else:
                h = out
    state.since += 1
    return out


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each fp64 value: 8 significant bits."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 256.0), e - 8)


def run_stack(st, steps: int | None = None, rebuild_every: int = 10, max_disp: float = 0.25):
    """Whole trajectory of a workloads.Stack-like object: outputs per step and the
    steps at which the lists were rebuilt."""
    cfgs = [wl.cfg for wl in st.layers]
    state = StackState([c.cutoff for c in cfgs], st.cfg.max_neighbors, rebuild_every, max_disp)
    outs = []
    T = len(st.traj) if steps is None else steps
    for t in range(T):
        outs.append(stack_step(state, st.traj[t], st.h0, st.layers, t, cfgs[0].storage))
    return outs, state.rebuilds
