"""ctypes binding of libe2v2.so: argument marshalling only.

Functions keep the C names.  Torch supplies device memory and the current HIP
stream; every step of the layer runs in the library's kernels.  Loading fails
loudly when the library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libe2v2.so")

E2V2_OK, E2V2_ERR_ARG, E2V2_ERR_CAPACITY, E2V2_ERR_UNSUPPORTED, E2V2_ERR_HIP = range(5)
E2V2_FP32, E2V2_BF16 = 0, 1

EXPORTS = [
    "e2v2_build_neighbors", "e2v2_build_neighbors_workspace_bytes", "e2v2_eaas_couple",
    "e2v2_attn_forward", "e2v2_attn_forward_taps", "e2v2_attn_prepare", "e2v2_attn_aggregate",
    "e2v2_attn_workspace_bytes", "e2v2_num_paths",
    "e2v2_path_table", "e2v2_eaas_coefficients", "e2v2_alignment_wigner", "e2v2_status_string",
    "e2v2_last_error", "e2v2_filter_neighbors", "e2v2_max_displacement2", "e2v2_stack_state_bytes",
    "e2v2_stack_workspace_bytes", "e2v2_stack_forward", "e2v2_layer_backward_workspace_bytes",
    "e2v2_layer_backward", "e2v2_stack_backward_workspace_bytes", "e2v2_stack_backward", "e2v2_attn_forward_noalloc",
    "e2v2_edge_forward", "e2v2_edge_workspace_bytes", "e2v2_edge_coefficients", "e2v2_target_order",
    "e2v2_target_order_workspace_bytes",
]


class LayerDesc(ctypes.Structure):
    _fields_ = [("lmax", ctypes.c_int32), ("channels", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("n_rbf", ctypes.c_int32), ("cutoff", ctypes.c_float), ("storage", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_q", ctypes.c_void_p), ("w_k", ctypes.c_void_p), ("w_v", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("w_rbf", ctypes.c_void_p), ("w_src", ctypes.c_void_p),
                ("w_tgt", ctypes.c_void_p)]


class Taps(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("hprime", ctypes.c_void_p), ("m", ctypes.c_void_p), ("hhat", ctypes.c_void_p),
                ("events", ctypes.c_void_p)]


class RebuildPolicy(ctypes.Structure):
    _fields_ = [("rebuild_every", ctypes.c_int32), ("max_displacement", ctypes.c_float),
                ("steps_since_rebuild", ctypes.c_int32), ("rebuilt", ctypes.c_int32), ("rebuilds", ctypes.c_int64)]


class E2V2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"e2v2 status {status}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m atomistic_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.e2v2_build_neighbors.argtypes = [vp, i32, f32, i32, vp, vp, vp, i64, ctypes.POINTER(i64), vp, vp, sz, vp]
    lib.e2v2_build_neighbors.restype = ctypes.c_int
    lib.e2v2_build_neighbors_workspace_bytes.argtypes = [i32, i32]
    lib.e2v2_build_neighbors_workspace_bytes.restype = sz
    lib.e2v2_target_order.argtypes = [vp, i32, vp, vp, sz, vp]
    lib.e2v2_target_order.restype = ctypes.c_int
    lib.e2v2_target_order_workspace_bytes.argtypes = [i32]
    lib.e2v2_target_order_workspace_bytes.restype = sz
    lib.e2v2_eaas_couple.argtypes = [vp, vp, ctypes.c_int, vp, i32, i32, i32, vp, ctypes.c_int, vp]
    lib.e2v2_eaas_couple.restype = ctypes.c_int
    lib.e2v2_attn_forward.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.POINTER(Weights), vp, vp, vp, vp,
                                      i32, vp, vp, sz, vp]
    lib.e2v2_attn_forward.restype = ctypes.c_int
    lib.e2v2_attn_forward_taps.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.POINTER(Weights), vp, vp, vp,
                                           vp, i32, vp, vp, sz, ctypes.POINTER(Taps), vp]
    lib.e2v2_attn_forward_taps.restype = ctypes.c_int
    lib.e2v2_attn_prepare.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.POINTER(Weights), i32, vp, sz, vp]
    lib.e2v2_attn_prepare.restype = ctypes.c_int
    lib.e2v2_attn_aggregate.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(Weights), vp, vp, vp, vp, i32, vp,
                                        vp, sz, vp]
    lib.e2v2_attn_aggregate.restype = ctypes.c_int
    lib.e2v2_attn_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), i32]
    lib.e2v2_attn_workspace_bytes.restype = sz
    lib.e2v2_num_paths.argtypes = [i32]
    lib.e2v2_num_paths.restype = i32
    lib.e2v2_path_table.argtypes = [i32, vp]
    lib.e2v2_path_table.restype = ctypes.c_int
    lib.e2v2_eaas_coefficients.argtypes = [i32, vp]
    lib.e2v2_eaas_coefficients.restype = ctypes.c_int
    lib.e2v2_alignment_wigner.argtypes = [i32, vp, vp]
    lib.e2v2_alignment_wigner.restype = ctypes.c_int
    lib.e2v2_filter_neighbors.argtypes = [vp, i32, f32, vp, vp, vp, vp, vp, vp]
    lib.e2v2_filter_neighbors.restype = ctypes.c_int
    lib.e2v2_max_displacement2.argtypes = [vp, vp, i32, vp, vp]
    lib.e2v2_max_displacement2.restype = ctypes.c_int
    lib.e2v2_stack_state_bytes.argtypes = [i32, ctypes.POINTER(LayerDesc), i32, i32]
    lib.e2v2_stack_state_bytes.restype = sz
    lib.e2v2_stack_workspace_bytes.argtypes = [i32, ctypes.POINTER(LayerDesc), i32, i32]
    lib.e2v2_stack_workspace_bytes.restype = sz
    lib.e2v2_stack_forward.argtypes = [i32, ctypes.POINTER(LayerDesc), ctypes.POINTER(Weights), vp, vp, i32, i32,
                                       ctypes.POINTER(RebuildPolicy), vp, sz, vp, vp, sz, vp]
    lib.e2v2_stack_forward.restype = ctypes.c_int
    lib.e2v2_layer_backward_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), i32, i64]
    lib.e2v2_layer_backward_workspace_bytes.restype = sz
    lib.e2v2_layer_backward.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.POINTER(Weights), vp, vp, vp, i64,
                                        i32, i32, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.e2v2_layer_backward.restype = ctypes.c_int
    lib.e2v2_stack_backward_workspace_bytes.argtypes = [i32, ctypes.POINTER(LayerDesc), i32, i32]
    lib.e2v2_stack_backward_workspace_bytes.restype = sz
    lib.e2v2_stack_backward.argtypes = [i32, ctypes.POINTER(LayerDesc), ctypes.POINTER(Weights), vp, vp, i32, i32,
                                        vp, sz, ctypes.POINTER(RebuildPolicy), vp, vp, vp, vp, sz, vp]
    lib.e2v2_stack_backward.restype = ctypes.c_int
    lib.e2v2_attn_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.POINTER(Weights), vp, vp, vp,
                                              vp, i32, vp, vp]
    lib.e2v2_attn_forward_noalloc.restype = ctypes.c_int
    lib.e2v2_edge_forward.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, ctypes.POINTER(Weights), vp, vp, vp, vp,
                                      i32, vp, vp, sz, vp]
    lib.e2v2_edge_forward.restype = ctypes.c_int
    lib.e2v2_edge_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), i32]
    lib.e2v2_edge_workspace_bytes.restype = sz
    lib.e2v2_edge_coefficients.argtypes = [i32, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double), i32]
    lib.e2v2_edge_coefficients.restype = i32
    lib.e2v2_status_string.argtypes = [ctypes.c_int]
    lib.e2v2_status_string.restype = ctypes.c_char_p
    lib.e2v2_last_error.argtypes = []
    lib.e2v2_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != E2V2_OK:
        raise E2V2Error(status, _lib.e2v2_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def storage_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return E2V2_FP32
    if dtype == torch.bfloat16:
        return E2V2_BF16
    raise ValueError(f"unsupported storage dtype {dtype}")


# ------------------------------------------------------------------ host tables
def e2v2_num_paths(lmax: int) -> int:
    return int(load().e2v2_num_paths(lmax))


def e2v2_path_table(lmax: int):
    import numpy as np
    n = e2v2_num_paths(lmax)
    if n < 0:
        raise ValueError("lmax out of range")
    t = np.zeros((n, 3), dtype=np.int32)
    _check(load().e2v2_path_table(lmax, t.ctypes.data))
    return [tuple(int(v) for v in row) for row in t]


def e2v2_eaas_coefficients(lmax: int):
    import numpy as np
    c = np.zeros((max(e2v2_num_paths(lmax), 1), 7), dtype=np.float32)
    _check(load().e2v2_eaas_coefficients(lmax, c.ctypes.data))
    return c


def e2v2_alignment_wigner(lmax: int, r):
    import numpy as np
    r = np.ascontiguousarray(r, dtype=np.float64)
    nd = sum((2 * l + 1) ** 2 for l in range(1, lmax + 1))
    d = np.zeros(max(nd, 1), dtype=np.float64)
    _check(load().e2v2_alignment_wigner(lmax, r.ctypes.data, d.ctypes.data))
    out, o = [], 0
    for l in range(1, lmax + 1):
        k = 2 * l + 1
        out.append(d[o:o + k * k].reshape(k, k).copy())
        o += k * k
    return out


# ------------------------------------------------------------------ device calls
def e2v2_build_neighbors(pos: torch.Tensor, cutoff: float, max_neighbors: int = 0, capacity: int | None = None,
                         workspace: torch.Tensor | None = None, stream=None, want_nnz: bool = True,
                         order_out: torch.Tensor | None = None):
    """Neighbour list of pos [n, 3] fp32 (device).  Returns (start, len, idx, nnz).
    order_out: optional int32 [n] device tensor receiving the targets' Hilbert-curve processing
    order (the permutation e2v2_target_order returns)."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    n = pos.shape[0]
    dev = pos.device
    start = torch.empty(n, dtype=torch.int32, device=dev)
    length = torch.empty(n, dtype=torch.int32, device=dev)
    wsb = int(lib.e2v2_build_neighbors_workspace_bytes(n, max_neighbors))
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    if max_neighbors > 0:
        cap = n * max_neighbors
    else:
        cap = capacity if capacity is not None else max(n * 64, 1)
    while True:
        idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        nnz = ctypes.c_int64(-1)
        st = lib.e2v2_build_neighbors(_ptr(pos), n, float(cutoff), max_neighbors, _ptr(start), _ptr(length),
                                      _ptr(idx), cap, ctypes.byref(nnz) if (want_nnz or max_neighbors == 0) else None,
                                      _ptr(order_out), _ptr(workspace), workspace.numel(), _stream(stream))
        if st == E2V2_ERR_CAPACITY and max_neighbors == 0:
            cap = int(nnz.value)
            continue
        _check(st)
        break
    if max_neighbors == 0:
        idx = idx[:int(nnz.value)]
    return start, length, idx, int(nnz.value)


def e2v2_target_order(pos: torch.Tensor, order: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Hilbert-curve processing order of pos [n, 3] fp32 (device) as an int32 [n]
    device tensor (written into `order` when given)."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    n = pos.shape[0]
    if order is None:
        order = torch.empty(n, dtype=torch.int32, device=pos.device)
    wsb = int(lib.e2v2_target_order_workspace_bytes(n))
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=pos.device)
    _check(lib.e2v2_target_order(_ptr(pos), n, _ptr(order), _ptr(workspace), workspace.numel(), _stream(stream)))
    return order


def e2v2_eaas_couple(pos: torch.Tensor, x: torch.Tensor, path_w: torch.Tensor, lmax: int,
                     out_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """y = sum_p w[p] (x (x) Y(r))_p via EAAS; x [n, (lmax+1)^2, C] fp32 or bf16."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    _dev(x, None, "x")
    _dev(path_w, torch.float32, "path_w")
    n, nc, C = x.shape
    if nc != (lmax + 1) ** 2:
        raise ValueError("x has the wrong number of components")
    y = torch.empty((n, nc, C), dtype=out_dtype, device=x.device)
    _check(lib.e2v2_eaas_couple(_ptr(pos), _ptr(x), storage_code(x.dtype), _ptr(path_w), n, lmax, C, _ptr(y),
                                storage_code(out_dtype), _stream(stream)))
    return y


def make_desc(lmax, channels, heads, n_rbf, cutoff, storage: torch.dtype) -> LayerDesc:
    return LayerDesc(lmax, channels, heads, n_rbf, float(cutoff), storage_code(storage))


def attn_workspace_bytes(desc: LayerDesc, n: int) -> int:
    return int(load().e2v2_attn_workspace_bytes(ctypes.byref(desc), n))


def e2v2_attn_forward(desc: LayerDesc, pos, h, weights: dict, nbr_start, nbr_len, nbr_idx, out=None,
                      workspace=None, taps: dict | None = None, stream=None,
                      target_order: torch.Tensor | None = None) -> torch.Tensor:
    """One layer forward.  weights: dict with w_q, w_k, w_v, w_o (storage dtype), w_rbf, w_src, w_tgt (fp32).
    taps: optional dict of preallocated device tensors among q, k, v, hprime, m, hhat, and
    "events": a list of 5 recorded-once torch.cuda.Event objects marking the stage boundaries."""
    lib = load()
    n = pos.shape[0]
    sdt = h.dtype
    for name in ("w_q", "w_k", "w_v", "w_o"):
        _dev(weights[name], sdt, name)
    for name in ("w_rbf", "w_src", "w_tgt"):
        _dev(weights[name], torch.float32, name)
    _dev(pos, torch.float32, "pos")
    _dev(h, sdt, "h")
    for t, nm in ((nbr_start, "nbr_start"), (nbr_len, "nbr_len"), (nbr_idx, "nbr_idx")):
        _dev(t, torch.int32, nm)
    if target_order is not None:
        _dev(target_order, torch.int32, "target_order")
    if out is None:
        out = torch.empty(h.shape, dtype=torch.float32, device=h.device)
    wsb = attn_workspace_bytes(desc, n)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=h.device)
    w = Weights(*(_ptr(weights[k]) for k in ("w_q", "w_k", "w_v", "w_o", "w_rbf", "w_src", "w_tgt")))
    if taps is None:
        st = lib.e2v2_attn_forward(ctypes.byref(desc), _ptr(pos), _ptr(h), ctypes.byref(w), _ptr(nbr_start),
                                   _ptr(nbr_len), _ptr(nbr_idx), _ptr(target_order), n, _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(stream))
    else:
        evs = taps.get("events")
        ev_arr = None
        if evs is not None:
            if len(evs) != 5:
                raise ValueError("events needs 5 entries")
            ev_arr = (ctypes.c_void_p * 5)(*(ctypes.c_void_p(e.cuda_event) for e in evs))
        tp = Taps(*(_ptr(taps.get(k)) for k in ("q", "k", "v", "hprime", "m", "hhat")),
                  ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
        st = lib.e2v2_attn_forward_taps(ctypes.byref(desc), _ptr(pos), _ptr(h), ctypes.byref(w), _ptr(nbr_start),
                                        _ptr(nbr_len), _ptr(nbr_idx), _ptr(target_order), n, _ptr(out),
                                        _ptr(workspace), workspace.numel(), ctypes.byref(tp), _stream(stream))
    _check(st)
    return out


def e2v2_attn_forward_noalloc(desc: LayerDesc, pos, h, weights: dict, nbr_start, nbr_len, nbr_idx, out: torch.Tensor,
                              stream=None, target_order: torch.Tensor | None = None) -> torch.Tensor:
    """e2v2_attn_forward with the library's own device array as workspace (no
    allocation in the call; `out` is the caller's)."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    _dev(h, h.dtype, "h")
    for t, nm in ((nbr_start, "nbr_start"), (nbr_len, "nbr_len"), (nbr_idx, "nbr_idx")):
        _dev(t, torch.int32, nm)
    if target_order is not None:
        _dev(target_order, torch.int32, "target_order")
    _dev(out, torch.float32, "out")
    w = _weights(weights, h.dtype)
    _check(lib.e2v2_attn_forward_noalloc(ctypes.byref(desc), _ptr(pos), _ptr(h), ctypes.byref(w), _ptr(nbr_start),
                                         _ptr(nbr_len), _ptr(nbr_idx), _ptr(target_order), pos.shape[0], _ptr(out),
                                         _stream(stream)))
    return out


def edge_workspace_bytes(desc: LayerDesc, n: int) -> int:
    return int(load().e2v2_edge_workspace_bytes(ctypes.byref(desc), n))


def e2v2_edge_forward(desc: LayerDesc, pos, h, weights: dict, w_edge, nbr_start, nbr_len, nbr_idx, out=None,
                      workspace=None, stream=None, target_order: torch.Tensor | None = None) -> torch.Tensor:
    """The exact edge-equivalent form (fp32 storage, l_max <= 2): weights as for the
    layer (w_q, w_k, w_v, w_o, w_rbf), w_edge [n_paths][C] fp32 the edge weights."""
    lib = load()
    n = pos.shape[0]
    _dev(pos, torch.float32, "pos")
    _dev(h, torch.float32, "h")
    _dev(w_edge, torch.float32, "w_edge")
    for t, nm in ((nbr_start, "nbr_start"), (nbr_len, "nbr_len"), (nbr_idx, "nbr_idx")):
        _dev(t, torch.int32, nm)
    if target_order is not None:
        _dev(target_order, torch.int32, "target_order")
    if out is None:
        out = torch.empty(h.shape, dtype=torch.float32, device=h.device)
    wsb = edge_workspace_bytes(desc, n)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=h.device)
    wd = dict(weights, w_src=w_edge, w_tgt=w_edge)
    w = _weights(wd, torch.float32)
    _check(lib.e2v2_edge_forward(ctypes.byref(desc), _ptr(pos), _ptr(h), ctypes.byref(w), _ptr(nbr_start),
                                 _ptr(nbr_len), _ptr(nbr_idx), _ptr(target_order), n, _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    return out


def _weights(weights: dict, sdt) -> Weights:
    for name in ("w_q", "w_k", "w_v", "w_o"):
        _dev(weights[name], sdt, name)
    for name in ("w_rbf", "w_src", "w_tgt"):
        _dev(weights[name], torch.float32, name)
    return Weights(*(_ptr(weights[k]) for k in ("w_q", "w_k", "w_v", "w_o", "w_rbf", "w_src", "w_tgt")))


def e2v2_attn_prepare(desc: LayerDesc, pos, h, weights: dict, workspace: torch.Tensor, stream=None):
    """Steps 2-3 of the layer into `workspace` (no neighbour list needed)."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    _dev(h, h.dtype, "h")
    w = _weights(weights, h.dtype)
    _check(lib.e2v2_attn_prepare(ctypes.byref(desc), _ptr(pos), _ptr(h), ctypes.byref(w), pos.shape[0],
                                 _ptr(workspace), workspace.numel(), _stream(stream)))


def e2v2_attn_aggregate(desc: LayerDesc, weights: dict, nbr_start, nbr_len, nbr_idx, out: torch.Tensor,
                        workspace: torch.Tensor, stream=None, target_order: torch.Tensor | None = None):
    """Steps 4-6 of the layer on a workspace that e2v2_attn_prepare filled; writes out."""
    lib = load()
    for t, nm in ((nbr_start, "nbr_start"), (nbr_len, "nbr_len"), (nbr_idx, "nbr_idx")):
        _dev(t, torch.int32, nm)
    if target_order is not None:
        _dev(target_order, torch.int32, "target_order")
    _dev(out, torch.float32, "out")
    w = _weights(weights, weights["w_q"].dtype)
    _check(lib.e2v2_attn_aggregate(ctypes.byref(desc), ctypes.byref(w), _ptr(nbr_start), _ptr(nbr_len),
                                   _ptr(nbr_idx), _ptr(target_order), nbr_start.shape[0], _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def backward_workspace_bytes(desc: LayerDesc, n: int, max_entries: int) -> int:
    return int(load().e2v2_layer_backward_workspace_bytes(ctypes.byref(desc), n, max_entries))


def e2v2_layer_backward(desc: LayerDesc, pos, h, weights: dict, nbr_start, nbr_len, nbr_idx, grad_out,
                        grad_h=None, workspace=None, stream=None,
                        target_order: torch.Tensor | None = None, grad_pos: torch.Tensor | None = None,
                        symmetric: bool = False, reuse_forward: bool = False):
    """dL/dh for L = sum(grad_out * layer(pos, h)) (any neighbour list); h and the
    projection weights in the storage dtype of desc, grad_out and the gradients fp32.
    With grad_pos (a [n, 3] fp32 device tensor) also dL/dpos; returns grad_h, or
    (grad_h, grad_pos) when grad_pos is given.  symmetric=True: the list is its own
    transpose (uncapped lists of e2v2_build_neighbors), so none is built.
    reuse_forward=True (fp32 storage): `workspace` holds what e2v2_attn_forward left
    in it for the same inputs (pass the same tensor to both), so q, k, v, h' are not
    recomputed."""
    lib = load()
    n = pos.shape[0]
    sdt = torch.bfloat16 if desc.storage == E2V2_BF16 else torch.float32
    _dev(pos, torch.float32, "pos")
    _dev(h, sdt, "h")
    _dev(grad_out, torch.float32, "grad_out")
    if tuple(grad_out.shape) != tuple(h.shape):
        raise ValueError(f"grad_out shape {tuple(grad_out.shape)} != h shape {tuple(h.shape)}")
    for t, nm in ((nbr_start, "nbr_start"), (nbr_len, "nbr_len"), (nbr_idx, "nbr_idx")):
        _dev(t, torch.int32, nm)
    if target_order is not None:
        _dev(target_order, torch.int32, "target_order")
    w = _weights(weights, sdt)
    if grad_h is None:
        grad_h = torch.empty(h.shape, dtype=torch.float32, device=h.device)
    _dev(grad_h, torch.float32, "grad_h")
    max_entries = nbr_idx.numel()
    wsb = backward_workspace_bytes(desc, n, max_entries)
    if workspace is None or workspace.numel() < wsb:
        if reuse_forward:
            raise ValueError("reuse_forward needs the workspace the forward ran on, of backward_workspace_bytes")
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=h.device)
    if grad_pos is not None:
        _dev(grad_pos, torch.float32, "grad_pos")
        if tuple(grad_pos.shape) != (n, 3):
            raise ValueError(f"grad_pos shape {tuple(grad_pos.shape)} != ({n}, 3)")
    _check(lib.e2v2_layer_backward(ctypes.byref(desc), _ptr(pos), _ptr(h), ctypes.byref(w), _ptr(nbr_start),
                                   _ptr(nbr_len), _ptr(nbr_idx), max_entries, int(bool(symmetric)),
                                   int(bool(reuse_forward)), _ptr(target_order),
                                   n, _ptr(grad_out),
                                   _ptr(grad_h), _ptr(grad_pos), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return grad_h if grad_pos is None else (grad_h, grad_pos)


# ------------------------------------------------------------------ neighbour reuse and the stack
def e2v2_filter_neighbors(pos, cutoff: float, nbr_start, nbr_len, nbr_idx, out_len=None, out_idx=None, stream=None):
    """Entries of each row within `cutoff` (same predicate as the builder), rows at the
    input's starts.  Returns (out_len, out_idx); pass nbr_len / nbr_idx to filter in place."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    for t, nm in ((nbr_start, "nbr_start"), (nbr_len, "nbr_len"), (nbr_idx, "nbr_idx")):
        _dev(t, torch.int32, nm)
    if out_len is None:
        out_len = torch.empty_like(nbr_len)
    if out_idx is None:
        out_idx = torch.empty_like(nbr_idx)
    _check(lib.e2v2_filter_neighbors(_ptr(pos), pos.shape[0], float(cutoff), _ptr(nbr_start), _ptr(nbr_len),
                                     _ptr(nbr_idx), _ptr(out_len), _ptr(out_idx), _stream(stream)))
    return out_len, out_idx


def e2v2_max_displacement2(pos, ref, out=None, stream=None) -> torch.Tensor:
    """Largest squared displacement (fp64) as a one-element device tensor."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    _dev(ref, torch.float32, "ref")
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=pos.device)
    _check(lib.e2v2_max_displacement2(_ptr(pos), _ptr(ref), pos.shape[0], _ptr(out), _stream(stream)))
    return out


class StackRun:
    """Device state and scratch of one e2v2_stack_forward run (allocated through torch),
    and the host rebuild policy the calls update."""

    def __init__(self, descs, weights, n: int, max_neighbors: int, device="cuda", rebuild_every: int = 10,
                 max_displacement: float = 0.25):
        lib = load()
        self.L = len(descs)
        self.descs = (LayerDesc * self.L)(*descs)
        self.sdt = weights[0]["w_q"].dtype
        self.weights = (Weights * self.L)(*(_weights(w, self.sdt) for w in weights))
        self._keep = weights                      # the weight tensors outlive the calls
        self.n, self.K = n, max_neighbors
        sb = int(lib.e2v2_stack_state_bytes(self.L, self.descs, n, max_neighbors))
        wb = int(lib.e2v2_stack_workspace_bytes(self.L, self.descs, n, max_neighbors))
        if sb == 0 or wb == 0:
            raise ValueError("invalid stack description")
        self.state = torch.empty(sb, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=device)
        self.policy = RebuildPolicy(rebuild_every, max_displacement, -1, 0, 0)

    def e2v2_stack_forward(self, pos, h, out=None, stream=None) -> torch.Tensor:
        lib = load()
        _dev(pos, torch.float32, "pos")
        _dev(h, self.sdt, "h")
        if out is None:
            out = torch.empty(h.shape, dtype=torch.float32, device=h.device)
        _dev(out, torch.float32, "out")
        _check(lib.e2v2_stack_forward(self.L, self.descs, self.weights, _ptr(pos), _ptr(h), self.n, self.K,
                                      ctypes.byref(self.policy), _ptr(self.state), self.state.numel(), _ptr(out),
                                      _ptr(self.workspace), self.workspace.numel(), _stream(stream)))
        return out

    def e2v2_stack_backward(self, pos, h, grad_out, grad_h=None, grad_pos=None, stream=None):
        """dL/dh (and dL/dpos if grad_pos, a [n, 3] fp32 tensor, is given) of L = sum(grad_out * out)
        for the output of the last e2v2_stack_forward call at (pos, h); h in the storage
        dtype, grad_out and the gradients fp32."""
        lib = load()
        if self.policy.rebuilds < 1:
            raise E2V2Error(E2V2_ERR_ARG, "e2v2_stack_backward: no e2v2_stack_forward call has filled the state")
        _dev(pos, torch.float32, "pos")
        _dev(h, self.sdt, "h")
        _dev(grad_out, torch.float32, "grad_out")
        if grad_h is None:
            grad_h = torch.empty(h.shape, dtype=torch.float32, device=h.device)
        if grad_pos is not None:
            _dev(grad_pos, torch.float32, "grad_pos")
        wb = int(lib.e2v2_stack_backward_workspace_bytes(self.L, self.descs, self.n, self.K))
        if wb == 0:
            raise ValueError("invalid stack description")
        if getattr(self, "bworkspace", None) is None or self.bworkspace.numel() < wb:
            self.bworkspace = torch.empty(wb, dtype=torch.uint8, device=h.device)
        _check(lib.e2v2_stack_backward(self.L, self.descs, self.weights, _ptr(pos), _ptr(h), self.n, self.K,
                                       _ptr(self.state), self.state.numel(), ctypes.byref(self.policy),
                                       _ptr(grad_out), _ptr(grad_h),
                                       _ptr(grad_pos), _ptr(self.bworkspace), self.bworkspace.numel(),
                                       _stream(stream)))
        return grad_h if grad_pos is None else (grad_h, grad_pos)
