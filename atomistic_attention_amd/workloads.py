"""Seeded synthetic workloads for the E2Former-V2 neighbour-attention layer.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the layer's arithmetic, so the fp64 oracle and the HIP path
can both consume its output without sharing any of the method.

Workload shapes follow the systems the pages measure on:
  * 1k / 10k / 100k atoms -- E2Former-V2 explainer, section 4.2, Table 3;
  * 32,768 atoms          -- same page, section 1.1, Figure 1;
  * neighbour cap K = 256 -- same page, section 3.2 (Figure 4a);
  * 5 A and 8 A cutoffs   -- Tessera article (short-range and long-range layers);
  * l_max = 2, 16 heads, 128 channels -- explainer, section 5.1 (recommended config);
  * a clustered system    -- Tessera article, the capsid-vs-solution imbalance.

No dataset item is used: positions are uniform (or block-uniform) random
points, features are N(0, 1), weights are N(0, 1)/sqrt(fan_in).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "Workload", "make_workload", "num_paths", "StackConfig", "STACKS",
           "Stack", "trajectory", "make_stack",
           "path_list", "round_bf16", "bf16_bits", "bf16_from_bits", "device_arrays"]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    n: int              # atoms
    geometry: str       # "uniform" or "blocks"
    density: float      # atoms / A^3 (background density for "blocks")
    cutoff: float       # A
    max_neighbors: int  # 0 = uncapped CSR, K > 0 = keep the K nearest
    lmax: int
    channels: int
    heads: int
    n_rbf: int
    storage: str        # "fp32" or "bf16"
    seed: int

    @property
    def n_comp(self) -> int:
        return (self.lmax + 1) ** 2


CONFIGS = {
    "c1": LayerConfig("c1", 256, "uniform", 0.1, 5.0, 0, 2, 32, 4, 8, "fp32", 1001),
    "c2": LayerConfig("c2", 1000, "uniform", 0.1, 5.0, 0, 2, 128, 16, 32, "fp32", 1002),
    "c3": LayerConfig("c3", 10000, "uniform", 0.1, 5.0, 0, 2, 128, 16, 32, "bf16", 1003),
    "c3b": LayerConfig("c3b", 10000, "uniform", 0.1, 5.0, 0, 3, 128, 16, 32, "bf16", 1003),
    "c4": LayerConfig("c4", 32768, "uniform", 0.1, 8.0, 256, 2, 128, 16, 32, "bf16", 1004),
    "c5": LayerConfig("c5", 100000, "blocks", 0.1, 8.0, 256, 2, 128, 16, 32, "bf16", 1005),
    # feature gradient: fp32 storage and an uncapped (symmetric) 5 A list, c4's atom count
    "g4": LayerConfig("g4", 32768, "uniform", 0.1, 5.0, 0, 2, 128, 16, 32, "fp32", 1006),
}

# Block model of the clustered system: the box is cut into 8^3 equal blocks;
# 154 of the 512 blocks (30.1 % of the volume) hold 0.15 atoms/A^3, the rest 0.10.
BLOCKS_PER_DIM = 8
DENSE_BLOCKS = 154
DENSE_DENSITY = 0.15


def path_list(lmax: int):
    """Canonical (l_in, l_filter, l_out) order: l_out outer, then l_in, then l_f.

    Every triple with |l_in - l_f| <= l_out <= l_in + l_f is kept (no parity
    selection), which is the order both the oracle and the library use for
    the per-path weight rows.  Pure index bookkeeping, no coefficients.
    """
    out = []
    for lo in range(lmax + 1):
        for li in range(lmax + 1):
            for lf in range(lmax + 1):
                if abs(li - lf) <= lo <= li + lf:
                    out.append((li, lf, lo))
    return out


def num_paths(lmax: int) -> int:
    return len(path_list(lmax))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns float64.

    Scaling by a power of two is exact, and numpy's round() is round-half-even,
    so this is a single correct rounding from fp64 (no fp32 double rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q = np.round(m * 256.0)                 # 8 significant bits
    return np.ldexp(q, e - 8)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of values already representable in bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Workload:
    """One layer invocation's inputs.

    Floating arrays are float64 holding exactly the values the GPU receives
    (already rounded to the storage dtype); ``pos`` holds fp32 values.
    """
    cfg: LayerConfig
    pos: np.ndarray     # [n, 3]  (fp32 values)
    h: np.ndarray       # [n, n_comp, C]
    w_q: np.ndarray     # [C, C]  (in, out)
    w_k: np.ndarray     # [C, C]
    w_v: np.ndarray     # [lmax+1, C, C]
    w_o: np.ndarray     # [lmax+1, C, C]
    w_rbf: np.ndarray   # [n_rbf, heads] fp32 values
    w_src: np.ndarray   # [n_paths, C] fp32 values
    w_tgt: np.ndarray   # [n_paths, C] fp32 values

    def storage_array(self, a: np.ndarray) -> np.ndarray:
        """The array as the device stores it: float32, or uint16 bf16 bits."""
        if self.cfg.storage == "bf16":
            return bf16_bits(a)
        return a.astype(np.float32)


def device_arrays(wl: Workload, device="cuda") -> dict:
    """Upload a workload as the library consumes it: positions, path weights and RBF
    weights fp32; features and projection weights in the storage dtype."""
    import torch

    dt = torch.bfloat16 if wl.cfg.storage == "bf16" else torch.float32

    def st(a):
        if dt == torch.bfloat16:
            return torch.from_numpy(np.ascontiguousarray(bf16_bits(a)).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    def f(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    return dict(pos=f(wl.pos), h=st(wl.h), dtype=dt,
                weights=dict(w_q=st(wl.w_q), w_k=st(wl.w_k), w_v=st(wl.w_v), w_o=st(wl.w_o),
                             w_rbf=f(wl.w_rbf), w_src=f(wl.w_src), w_tgt=f(wl.w_tgt)))


def _box_side(cfg: LayerConfig) -> float:
    if cfg.geometry == "uniform":
        return (cfg.n / cfg.density) ** (1.0 / 3.0)
    frac = DENSE_BLOCKS / BLOCKS_PER_DIM ** 3
    mean_density = frac * DENSE_DENSITY + (1.0 - frac) * cfg.density
    return (cfg.n / mean_density) ** (1.0 / 3.0)


def _dense_blocks(rng: np.random.Generator) -> np.ndarray:
    """Which of the 8^3 blocks are dense: the first draw of the workload's generator."""
    dense = np.zeros(BLOCKS_PER_DIM ** 3, dtype=bool)
    dense[rng.permutation(BLOCKS_PER_DIM ** 3)[:DENSE_BLOCKS]] = True
    return dense


def dense_block_mask(wl) -> np.ndarray:
    """For a block-geometry workload: True for the atoms that lie in a dense block."""
    cfg = wl.cfg
    if cfg.geometry != "blocks":
        return np.zeros(cfg.n, dtype=bool)
    dense = _dense_blocks(np.random.default_rng(cfg.seed))
    nb = BLOCKS_PER_DIM
    side = _box_side(cfg)
    bi = np.clip(np.floor((np.asarray(wl.pos) + 0.5 * side) / (side / nb)).astype(np.int64), 0, nb - 1)
    return dense[(bi[:, 0] * nb + bi[:, 1]) * nb + bi[:, 2]]


def _positions(cfg: LayerConfig, rng: np.random.Generator, n: int) -> np.ndarray:
    side = _box_side(cfg)
    if cfg.geometry == "uniform":
        p = rng.uniform(-0.5 * side, 0.5 * side, size=(n, 3))
        return p.astype(np.float32).astype(np.float64)
    nb = BLOCKS_PER_DIM
    nblk = nb ** 3
    bside = side / nb
    dense = _dense_blocks(rng)
    dens = np.where(dense, DENSE_DENSITY, cfg.density)
    expect = dens * bside ** 3
    expect = expect * (n / expect.sum())
    counts = np.floor(expect).astype(np.int64)
    rem = n - counts.sum()
    order = np.argsort(-(expect - counts), kind="stable")
    counts[order[:rem]] += 1
    blk = np.repeat(np.arange(nblk), counts)
    bi = np.stack([blk // (nb * nb), (blk // nb) % nb, blk % nb], axis=1).astype(np.float64)
    u = rng.uniform(0.0, 1.0, size=(n, 3))
    p = (bi + u) * bside - 0.5 * side
    p = p[rng.permutation(n)]          # user order carries no spatial structure
    return p.astype(np.float32).astype(np.float64)


def make_workload(cfg: LayerConfig | str, n: int | None = None, seed: int | None = None) -> Workload:
    """Draw a workload.  ``n`` overrides the atom count (same density / box rule)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if n is not None or seed is not None:
        cfg = dataclasses.replace(cfg, n=cfg.n if n is None else n, seed=cfg.seed if seed is None else seed)
    rng = np.random.default_rng(cfg.seed)
    N, C, L = cfg.n, cfg.channels, cfg.lmax
    nc = (L + 1) ** 2
    paths = path_list(L)
    pos = _positions(cfg, rng, N)
    rnd = round_bf16 if cfg.storage == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    h = rnd(rng.standard_normal((N, nc, C)))
    w_q = rnd(rng.standard_normal((C, C)) / math.sqrt(C))
    w_k = rnd(rng.standard_normal((C, C)) / math.sqrt(C))
    w_v = rnd(rng.standard_normal((L + 1, C, C)) / math.sqrt(C))
    w_o = rnd(rng.standard_normal((L + 1, C, C)) / math.sqrt(C))
    w_rbf = f32(rng.standard_normal((cfg.n_rbf, cfg.heads)) / math.sqrt(cfg.n_rbf))
    fan = {lo: sum(1 for p in paths if p[2] == lo) for lo in range(L + 1)}
    scale = np.array([1.0 / math.sqrt(fan[p[2]]) for p in paths])[:, None]
    w_src = f32(rng.standard_normal((len(paths), C)) * scale)
    w_tgt = f32(rng.standard_normal((len(paths), C)) * scale)
    return Workload(cfg, pos, h, w_q, w_k, w_v, w_o, w_rbf, w_src, w_tgt)


# ---------------------------------------------------------------------------
# Four-layer stacks over a moving system (Tessera article: three short-range
# layers with a 5 A cutoff and one long-range layer with 8 A; neighbour lists
# rebuilt every 10 steps, early when an atom has moved more than 0.25 A).


@dataclasses.dataclass(frozen=True)
class StackConfig:
    name: str
    base: str           # LayerConfig giving geometry, density, l_max, C, heads, n_rbf, storage
    n: int
    cutoffs: tuple      # per layer, in order (A)
    max_neighbors: int  # K of the list at the largest cutoff
    seed: int
    steps: int          # trajectory length
    sigma: float        # per-step random displacement, per coordinate (A)


STACKS = {
    "s1": StackConfig("s1", "c1", 256, (5.0, 5.0, 5.0, 8.0), 256, 2001, 16, 0.005),
    "s2": StackConfig("s2", "c3", 2000, (5.0, 5.0, 5.0, 8.0), 256, 2002, 3, 0.005),
    "s4": StackConfig("s4", "c4", 32768, (5.0, 5.0, 5.0, 8.0), 256, 2004, 100, 0.005),
}


@dataclasses.dataclass
class Stack:
    """Inputs of a stack run: one weight set per layer (each a Workload whose
    cutoff is the layer's), the features h0 fed to the first layer at every
    step, and positions per step (fp32 values)."""
    cfg: StackConfig
    layers: list
    h0: np.ndarray
    traj: list

    @property
    def base(self) -> LayerConfig:
        return self.layers[0].cfg


def trajectory(pos0: np.ndarray, steps: int, sigma: float, seed: int, jumps=()) -> list:
    """Positions for ``steps`` steps: a random walk with N(0, sigma^2) steps per
    coordinate, each step rounded to fp32; ``jumps`` adds (step, atom, (dx, dy, dz))
    offsets at the given steps (kept in later steps)."""
    rng = np.random.default_rng(seed)
    p = np.asarray(pos0, dtype=np.float64).astype(np.float32).astype(np.float64)
    out = [p.copy()]
    for t in range(1, steps):
        p = p + rng.standard_normal(p.shape) * sigma
        for (js, a, v) in jumps:
            if js == t:
                p[a] = p[a] + np.asarray(v, dtype=np.float64)
        p = p.astype(np.float32).astype(np.float64)
        out.append(p.copy())
    return out


def make_stack(cfg: StackConfig | str, n: int | None = None, steps: int | None = None, jumps=()) -> Stack:
    """Draw a stack: layer l's weights come from the base config with the layer's
    cutoff and seed + l; the trajectory starts at the base geometry."""
    if isinstance(cfg, str):
        cfg = STACKS[cfg]
    if n is not None or steps is not None:
        cfg = dataclasses.replace(cfg, n=cfg.n if n is None else n, steps=cfg.steps if steps is None else steps)
    base = dataclasses.replace(CONFIGS[cfg.base], n=cfg.n, max_neighbors=cfg.max_neighbors)
    layers = [make_workload(dataclasses.replace(base, cutoff=rc, seed=cfg.seed + l)) for l, rc in enumerate(cfg.cutoffs)]
    # the first layer's draw supplies the start geometry and h0
    pos0, h0 = layers[0].pos, layers[0].h
    traj = trajectory(pos0, cfg.steps, cfg.sigma, cfg.seed + 1000, jumps)
    return Stack(cfg, layers, h0, traj)
