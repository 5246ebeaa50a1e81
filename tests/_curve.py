"""Test-side reference of the targets' Hilbert-curve processing order, in numpy.

The curve is J. Skilling's construction ("Programming the Hilbert curve", AIP
Conf. Proc. 707, 2004): axes to the transposed form of the index (undo the
excess work level by level, then a Gray code), bits read from the top level
down, first axis first.  The cell grid follows the rule stated with
e2v2_target_order in include/e2v2.h.  Written independently of the library
(vectorised over atoms); the CPU tests pin it by properties that any Hilbert
curve has and a wrong bit order or exchange step breaks."""
import numpy as np

BITS = 10


def hilbert_index(q: np.ndarray, bits: int = BITS) -> np.ndarray:
    """[m, 3] non-negative ints below 2^bits -> [m] Hilbert indices (3 bits per level)."""
    X = [q[:, a].astype(np.int64).copy() for a in range(3)]
    Q = 1 << (bits - 1)
    while Q > 1:
        P = Q - 1
        for i in range(3):
            hit = (X[i] & Q) != 0
            flip = np.where(hit, X[0] ^ P, X[0])
            t = np.where(hit, 0, (X[0] ^ X[i]) & P)
            X[0] = flip ^ t
            if i:
                X[i] = X[i] ^ t
        Q >>= 1
    X[1] ^= X[0]
    X[2] ^= X[1]
    t = np.zeros_like(X[0])
    Q = 1 << (bits - 1)
    while Q > 1:
        t = np.where((X[2] & Q) != 0, t ^ (Q - 1), t)
        Q >>= 1
    for i in range(3):
        X[i] ^= t
    key = np.zeros(len(q), dtype=np.int64)
    for j in range(bits - 1, -1, -1):
        for i in range(3):
            key = (key << 1) | ((X[i] >> j) & 1)
    return key


def cells(pos: np.ndarray) -> np.ndarray:
    """[n, 3] fp32 positions -> [n, 3] cell coordinates of the curve's grid."""
    pos = np.asarray(pos, dtype=np.float32)
    n = len(pos)
    fin = np.isfinite(pos)
    lo = np.where(fin, pos, np.float32(np.inf)).min(axis=0)
    hi = np.where(fin, pos, np.float32(-np.inf)).max(axis=0)
    with np.errstate(invalid="ignore", over="ignore"):
        ext = (hi - lo).astype(np.float32)
    mx = np.float32(max(0.0, float(np.nanmax(np.where(np.isnan(ext), -np.inf, ext)))))
    lo = np.where(np.isfinite(lo), lo, np.float32(0)).astype(np.float32)
    inv = np.float32(0.0)
    if mx > 0 and np.isfinite(mx):
        fl = np.float32(mx * np.float32(2.0 ** -10))
        V = (float(max(ext[0], fl)) * float(max(ext[1], fl))) * float(max(ext[2], fl))
        E = int(np.frexp(V / (8.0 * n))[1])
        k = max((E - 1) // 3, -126)
        while k < 127 and np.float32(mx * np.float32(2.0 ** -k)) >= np.float32(1023.0):
            k += 1
        inv = np.float32(2.0 ** -k)
    with np.errstate(invalid="ignore", over="ignore"):
        c = ((pos - lo[None, :]).astype(np.float32) * inv).astype(np.float32)
    q = np.where(c >= 1023.0, 1023.0, np.where(c > 0.0, np.floor(c), 0.0))
    return q.astype(np.int64)


def target_order(pos: np.ndarray) -> np.ndarray:
    """The permutation e2v2_target_order returns: atoms by Hilbert index, ties by id."""
    key = hilbert_index(cells(pos))
    return np.argsort(key, kind="stable").astype(np.int32)
