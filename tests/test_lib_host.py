"""Host-side checks of the HIP library that need no GPU: it loads, exports every
symbol include/e2v2.h declares, its tables agree with the oracle, and argument
errors are reported before anything is enqueued."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from atomistic_attention_amd import binding as B
from atomistic_attention_amd import workloads as W
from oracle import so3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: errors come first
FAKE_MIS = ctypes.c_void_p(0x10004)


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "e2v2.h")).read()
    declared = set(re.findall(r"\b(e2v2_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_path_table_matches(lib):
    for L in range(4):
        assert B.e2v2_path_table(L) == so3.paths(L) == W.path_list(L)
        assert B.e2v2_num_paths(L) == len(so3.paths(L))
    assert B.e2v2_num_paths(4) == -1


def test_eaas_coefficients_match_oracle(lib):
    for L in range(4):
        c = B.e2v2_eaas_coefficients(L)
        for p, (li, lf, lo) in enumerate(so3.paths(L)):
            E = math.sqrt(2 * lf + 1) * so3.coupling_tensor(li, lf, lo)[:, lf, :]
            odd = (li + lf + lo) % 2 == 1
            for mo in range(-lo, lo + 1):
                mi = -mo if odd else mo
                ref = E[mi + li, mo + lo] if abs(mi) <= li else 0.0
                assert abs(c[p, mo + lo] - ref) < 3e-7, (L, li, lf, lo, mo)


def test_alignment_wigner_matches_oracle(lib):
    rng = np.random.default_rng(8)
    for r in list(rng.standard_normal((6, 3))) + [np.array([0, 0, -3.0]), np.array([0, 0, 1e-3])]:
        D = B.e2v2_alignment_wigner(3, r)
        R = so3.alignment_rotation(r)
        for l in range(1, 4):
            assert np.max(np.abs(D[l - 1] - so3.wigner_d(R, l))) < 1e-12


def _desc(**kw):
    d = dict(lmax=2, channels=128, heads=16, n_rbf=32, cutoff=5.0, storage=B.E2V2_BF16)
    d.update(kw)
    return B.LayerDesc(d["lmax"], d["channels"], d["heads"], d["n_rbf"], d["cutoff"], d["storage"])


def _attn(lib, desc, n=10, ws_bytes=None, ptr=FAKE, weights=None):
    w = weights or B.Weights(*([ptr] * 7))
    if ws_bytes is not None:
        wsb = ws_bytes
    elif desc is not None:
        wsb = lib.e2v2_attn_workspace_bytes(ctypes.byref(desc), max(n, 0))
    else:
        wsb = 1 << 20
    return lib.e2v2_attn_forward(ctypes.byref(desc) if desc is not None else None, ptr, ptr, ctypes.byref(w),
                                 ptr, ptr, ptr, None, n, ptr, ptr, wsb, None)


def test_attn_argument_errors(lib):
    assert _attn(lib, None) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(lmax=4)) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(lmax=-1)) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(channels=100)) == B.E2V2_ERR_ARG          # not a multiple of heads
    assert _attn(lib, _desc(channels=256)) == B.E2V2_ERR_UNSUPPORTED  # 16 channels per head
    assert _attn(lib, _desc(channels=16, heads=2)) == B.E2V2_ERR_UNSUPPORTED
    assert _attn(lib, _desc(n_rbf=1)) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(n_rbf=65)) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(cutoff=0.0)) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(cutoff=float("nan"))) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(storage=7)) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(), n=-1) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(), ptr=FAKE_MIS) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(), ptr=None) == B.E2V2_ERR_ARG
    assert _attn(lib, _desc(), ws_bytes=100) == B.E2V2_ERR_ARG
    assert "workspace" in lib.e2v2_last_error().decode()
    assert _attn(lib, _desc(), n=0) == B.E2V2_OK                       # nothing to do


def test_split_forward_argument_errors(lib):
    """The two halves check what they use; argument errors enqueue nothing."""
    d = _desc()
    wsb = lib.e2v2_attn_workspace_bytes(ctypes.byref(d), 10)
    full = B.Weights(*([FAKE] * 7))
    prep = lambda desc=d, n=10, pos=FAKE, h=FAKE, w=full, ws=FAKE, b=wsb: lib.e2v2_attn_prepare(
        ctypes.byref(desc) if desc is not None else None, pos, h, ctypes.byref(w), n, ws, b, None)
    agg = lambda desc=d, n=10, nbr=FAKE, out=FAKE, w=full, ws=FAKE, b=wsb: lib.e2v2_attn_aggregate(
        ctypes.byref(desc) if desc is not None else None, ctypes.byref(w), nbr, nbr, nbr, None, n, out, ws, b, None)
    for call in (prep, agg):
        assert call(desc=None) == B.E2V2_ERR_ARG
        assert call(desc=_desc(lmax=4)) == B.E2V2_ERR_ARG
        assert call(n=-1) == B.E2V2_ERR_ARG
        assert call(ws=None) == B.E2V2_ERR_ARG
        assert call(b=100) == B.E2V2_ERR_ARG
        assert call(n=0) == B.E2V2_OK
    assert prep(pos=None) == B.E2V2_ERR_ARG and prep(h=FAKE_MIS) == B.E2V2_ERR_ARG
    assert agg(nbr=None) == B.E2V2_ERR_ARG and agg(out=FAKE_MIS) == B.E2V2_ERR_ARG
    # prepare does not need the attention weights, aggregate does not need the projection ones
    no_rbf = B.Weights(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE)
    no_q = B.Weights(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert agg(w=no_rbf) == B.E2V2_ERR_ARG
    assert prep(w=no_q) == B.E2V2_ERR_ARG


def test_workspace_sizes(lib):
    d = _desc()
    a, b = lib.e2v2_attn_workspace_bytes(ctypes.byref(d), 1000), lib.e2v2_attn_workspace_bytes(ctypes.byref(d), 2000)
    assert 0 < a < b
    # bf16 storage: q and k fp32, h' in fp16, D blocks, padded positions, the message m
    # in fp16 and its node scale (v is projected and coupled in registers, never stored)
    per_node = 128 * 4 + 128 * 4 + 9 * 128 * 2 + 34 * 4 + 16 + 9 * 128 * 2 + 4
    assert abs((b - a) / 1000 - per_node) < 2
    # fp32 storage adds v and stores h' in fp32
    d32 = _desc(storage=B.E2V2_FP32)
    a, b = lib.e2v2_attn_workspace_bytes(ctypes.byref(d32), 1000), lib.e2v2_attn_workspace_bytes(ctypes.byref(d32), 2000)
    per_node = 128 * 4 * 2 + 9 * 128 * 4 + 9 * 128 * 4 + 34 * 4 + 16 + 9 * 128 * 4
    assert abs((b - a) / 1000 - per_node) < 2
    assert lib.e2v2_build_neighbors_workspace_bytes(1000, 0) > 0


def test_neighbor_argument_errors(lib):
    nnz = ctypes.c_int64(0)
    ws = lib.e2v2_build_neighbors_workspace_bytes(100, 16)
    call = lambda n=100, rc=5.0, K=16, cap=1600, nz=ctypes.byref(nnz), wsb=ws, ptr=FAKE: lib.e2v2_build_neighbors(
        ptr, n, rc, K, ptr, ptr, ptr, cap, nz, None, ptr, wsb, None)
    assert call(n=-1) == B.E2V2_ERR_ARG
    assert call(rc=0.0) == B.E2V2_ERR_ARG
    assert call(rc=float("inf")) == B.E2V2_ERR_ARG
    assert call(K=-2) == B.E2V2_ERR_ARG
    assert call(K=5000) == B.E2V2_ERR_ARG
    assert call(K=0, nz=None) == B.E2V2_ERR_ARG
    assert call(cap=1599) == B.E2V2_ERR_ARG
    assert call(wsb=10) == B.E2V2_ERR_ARG
    assert call(ptr=FAKE_MIS) == B.E2V2_ERR_ARG
    assert call(n=0) == B.E2V2_OK and nnz.value == 0


def test_target_order_argument_errors(lib):
    ws = lib.e2v2_target_order_workspace_bytes(1000)
    assert ws >= 3 * 4 * 1000 and lib.e2v2_target_order_workspace_bytes(2000) > ws
    assert lib.e2v2_target_order_workspace_bytes(-1) == 0
    call = lambda n=1000, pos=FAKE, order=FAKE, w=FAKE, wsb=ws: lib.e2v2_target_order(pos, n, order, w, wsb, None)
    assert call(n=-1) == B.E2V2_ERR_ARG
    assert call(n=2 ** 31 - 1) == B.E2V2_ERR_ARG
    assert call(pos=None) == B.E2V2_ERR_ARG
    assert call(order=None) == B.E2V2_ERR_ARG
    assert call(w=None) == B.E2V2_ERR_ARG
    assert call(pos=ctypes.c_void_p(0x10002)) == B.E2V2_ERR_ARG
    assert call(wsb=ws - 1) == B.E2V2_ERR_ARG
    assert call(n=0, pos=None, order=None, w=None, wsb=0) == B.E2V2_OK


def test_eaas_argument_errors(lib):
    f = lambda L=2, C=128, dt=0, n=10, ptr=FAKE: lib.e2v2_eaas_couple(ptr, ptr, dt, ptr, n, L, C, ptr, 0, None)
    assert f(L=4) == B.E2V2_ERR_ARG
    assert f(C=12) == B.E2V2_ERR_ARG
    assert f(C=512) == B.E2V2_ERR_ARG
    assert f(dt=3) == B.E2V2_ERR_ARG
    assert f(n=-1) == B.E2V2_ERR_ARG
    assert f(ptr=FAKE_MIS) == B.E2V2_ERR_ARG
    assert f(n=0) == B.E2V2_OK


def test_status_strings(lib):
    assert lib.e2v2_status_string(0) == b"ok"
    assert lib.e2v2_status_string(2) == b"insufficient neighbour capacity"


def test_reuse_argument_errors(lib):
    """Neighbour filter and displacement: argument errors come before any launch."""
    flt = lambda n=10, rc=5.0, pos=FAKE, p=FAKE: lib.e2v2_filter_neighbors(pos, n, rc, p, p, p, p, p, None)
    assert flt(n=-1) == B.E2V2_ERR_ARG and flt(rc=0.0) == B.E2V2_ERR_ARG and flt(rc=float("inf")) == B.E2V2_ERR_ARG
    assert flt(pos=None) == B.E2V2_ERR_ARG and flt(p=FAKE_MIS) == B.E2V2_ERR_ARG
    assert flt(n=0) == B.E2V2_OK
    dsp = lambda n=10, pos=FAKE, out=FAKE: lib.e2v2_max_displacement2(pos, pos, n, out, None)
    assert dsp(n=-1) == B.E2V2_ERR_ARG and dsp(pos=None) == B.E2V2_ERR_ARG and dsp(out=None) == B.E2V2_ERR_ARG
    assert dsp(pos=FAKE_MIS) == B.E2V2_ERR_ARG


def test_stack_argument_errors(lib):
    """The stack checks layer shapes, K, the policy and buffer sizes before anything
    runs, and leaves the policy unchanged on an error."""
    descs = (B.LayerDesc * 4)(*[_desc(cutoff=c) for c in (5.0, 5.0, 5.0, 8.0)])
    ws = (B.Weights * 4)(*[B.Weights(*([FAKE] * 7)) for _ in range(4)])
    n, K = 10, 16
    sb = lib.e2v2_stack_state_bytes(4, descs, n, K)
    wb = lib.e2v2_stack_workspace_bytes(4, descs, n, K)
    assert sb > 0 and wb > 0
    pol = B.RebuildPolicy(10, 0.25, -1, 0, 0)

    def call(L=4, d=descs, w=ws, n=n, K=K, policy=pol, state=FAKE, s=sb, out=FAKE, work=FAKE, b=wb):
        return lib.e2v2_stack_forward(L, d, w, FAKE, FAKE, n, K, ctypes.byref(policy) if policy is not None else None,
                                      state, s, out, work, b, None)
    assert call(L=0) == B.E2V2_ERR_ARG and call(L=17) == B.E2V2_ERR_ARG
    assert call(K=0) == B.E2V2_ERR_ARG and call(K=5000) == B.E2V2_ERR_ARG
    assert call(policy=None) == B.E2V2_ERR_ARG
    assert call(policy=B.RebuildPolicy(0, 0.25, -1, 0, 0)) == B.E2V2_ERR_ARG
    assert call(policy=B.RebuildPolicy(10, float("nan"), -1, 0, 0)) == B.E2V2_ERR_ARG
    assert call(s=sb - 1) == B.E2V2_ERR_ARG and call(b=wb - 1) == B.E2V2_ERR_ARG
    assert call(state=None) == B.E2V2_ERR_ARG and call(out=FAKE_MIS) == B.E2V2_ERR_ARG
    mixed = (B.LayerDesc * 2)(_desc(), _desc(lmax=1))
    assert call(L=2, d=mixed) == B.E2V2_ERR_ARG
    bad = (B.LayerDesc * 2)(_desc(), _desc(heads=3))
    assert call(L=2, d=bad) != B.E2V2_OK
    assert (pol.steps_since_rebuild, pol.rebuilt, pol.rebuilds) == (-1, 0, 0)
    assert call(n=0) == B.E2V2_OK
    # one distinct cutoff needs one list, two need two
    one = (B.LayerDesc * 2)(_desc(cutoff=5.0), _desc(cutoff=5.0))
    two = (B.LayerDesc * 2)(_desc(cutoff=5.0), _desc(cutoff=8.0))
    assert lib.e2v2_stack_state_bytes(2, two, 1000, 64) - lib.e2v2_stack_state_bytes(2, one, 1000, 64) >= 1000 * 65 * 4


def _bwd(lib, desc, n=10, ws_bytes=None, ptr=FAKE, gpos=None, entries=100, reuse=0):
    w = B.Weights(*([ptr] * 7))
    wsb = ws_bytes if ws_bytes is not None else lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(desc),
                                                                                       max(n, 0), entries)
    return lib.e2v2_layer_backward(ctypes.byref(desc), ptr, ptr, ctypes.byref(w), ptr, ptr, ptr, entries, 0, reuse,
                                   None, n, ptr, ptr, gpos, ptr, wsb, None)


def test_backward_argument_errors_and_workspace(lib):
    d32 = _desc(storage=B.E2V2_FP32)
    # bf16 storage: a bf16 forward keeps h' in fp16, so its workspace cannot be reused
    assert _bwd(lib, _desc(), reuse=1) == B.E2V2_ERR_UNSUPPORTED
    assert "fp32" in lib.e2v2_last_error().decode()
    assert _bwd(lib, _desc(), ws_bytes=100) == B.E2V2_ERR_ARG
    # bf16 storage widens h (n x 9 x 128 fp32) and W_Q, W_K, W_V[0..2], W_O[0..2] (8 x 128 x 128 fp32)
    # into the workspace of the fp32 gradient
    for n in (1000, 2000):
        extra = (lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(_desc()), n, 0)
                 - lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(d32), n, 0))
        assert abs(extra - (n * 9 * 128 * 4 + 8 * 128 * 128 * 4)) <= 5 * 256
    assert _bwd(lib, _desc(storage=B.E2V2_FP32, channels=256)) == B.E2V2_ERR_UNSUPPORTED
    assert _bwd(lib, d32, n=-1) == B.E2V2_ERR_ARG
    assert _bwd(lib, d32, ptr=None) == B.E2V2_ERR_ARG
    assert _bwd(lib, d32, ptr=FAKE_MIS) == B.E2V2_ERR_ARG
    assert _bwd(lib, d32, ws_bytes=100) == B.E2V2_ERR_ARG
    assert "workspace" in lib.e2v2_last_error().decode()
    assert _bwd(lib, d32, gpos=FAKE_MIS) == B.E2V2_ERR_ARG
    assert _bwd(lib, d32, entries=-1, ws_bytes=1 << 30) == B.E2V2_ERR_ARG
    assert _bwd(lib, d32, entries=1 << 31, ws_bytes=1 << 30) == B.E2V2_ERR_ARG
    assert _bwd(lib, d32, n=0) == B.E2V2_OK
    # the forward's fp32 workspace plus dL/dh', dL/dhhat, dL/dm, m, three per-head
    # values, dq, dk and four counters of the transposed list per node
    fa = lib.e2v2_attn_workspace_bytes(ctypes.byref(d32), 2000) - lib.e2v2_attn_workspace_bytes(ctypes.byref(d32), 1000)
    ba = (lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(d32), 2000, 0)
          - lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(d32), 1000, 0))
    assert abs((ba - fa) / 1000 - (4 * 9 * 128 * 4 + 3 * 16 * 4 + 2 * 128 * 4 + 4 * 4)) < 2
    # plus 4 bytes per list entry for the transposed list
    e0 = lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(d32), 1000, 0)
    assert abs(lib.e2v2_layer_backward_workspace_bytes(ctypes.byref(d32), 1000, 100000) - e0 - 400000) <= 256


def test_stack_backward_argument_errors(lib):
    descs = (B.LayerDesc * 2)(_desc(), _desc())                        # bf16 storage
    w = (B.Weights * 2)(B.Weights(*([FAKE] * 7)), B.Weights(*([FAKE] * 7)))
    pol = ctypes.byref(B.RebuildPolicy(10, 0.25, 1, 1, 1))            # as left by one forward call
    st = lib.e2v2_stack_backward(2, descs, w, FAKE, FAKE, 10, 8, FAKE, 1 << 20, pol, FAKE, FAKE, None, FAKE, 100,
                                 None)
    assert st == B.E2V2_ERR_ARG and "workspace" in lib.e2v2_last_error().decode()
    d32 = (B.LayerDesc * 2)(_desc(storage=B.E2V2_FP32), _desc(storage=B.E2V2_FP32, cutoff=8.0))
    st = lib.e2v2_stack_backward(2, d32, w, FAKE, FAKE, 10, 8, FAKE, 1 << 20, pol, FAKE, FAKE, FAKE_MIS, FAKE,
                                 1 << 30, None)
    assert st == B.E2V2_ERR_ARG
    st = lib.e2v2_stack_backward(2, d32, w, FAKE, FAKE, 10, 8, FAKE, 1 << 20, pol, FAKE, FAKE, None, FAKE, 100, None)
    assert st == B.E2V2_ERR_ARG and "workspace" in lib.e2v2_last_error().decode()
    # no forward call yet: the state holds no lists, so nothing may run
    for fresh in (B.RebuildPolicy(10, 0.25, -1, 0, 0), None):
        st = lib.e2v2_stack_backward(2, d32, w, FAKE, FAKE, 10, 8, FAKE, 1 << 20,
                                     ctypes.byref(fresh) if fresh else None, FAKE, FAKE, None, FAKE, 1 << 30, None)
        assert st == B.E2V2_ERR_ARG
    assert "e2v2_stack_forward" in lib.e2v2_last_error().decode() or "policy" in lib.e2v2_last_error().decode()
    assert lib.e2v2_stack_backward_workspace_bytes(2, d32, 1000, 8) > lib.e2v2_layer_backward_workspace_bytes(
        ctypes.byref(d32[0]), 1000, 8000)


def test_stack_backward_workspace_has_one_transposed_list_per_cutoff(lib):
    """Layers 5, 5, 5, 8 A share two distinct lists: the gradient's workspace holds
    two transposed lists, not four (4 bytes per entry of an n x K list each)."""
    f = B.E2V2_FP32
    four = (B.LayerDesc * 4)(*[_desc(storage=f, cutoff=c) for c in (5.0, 5.0, 5.0, 8.0)])
    two = (B.LayerDesc * 4)(*[_desc(storage=f, cutoff=c) for c in (5.0, 6.0, 7.0, 8.0)])
    n, K = 4096, 256
    a = lib.e2v2_stack_backward_workspace_bytes(4, four, n, K)
    b = lib.e2v2_stack_backward_workspace_bytes(4, two, n, K)
    assert b - a >= 2 * n * K * 4 and b - a <= 2 * (n * K * 4 + 5 * (n + 1) * 4 + 5 * 256)


def test_noalloc_forward_rejects_sizes_beyond_its_array(lib):
    """The allocation-free forward refuses, before any HIP call, an input whose
    workspace exceeds its 64 MiB device array; argument errors come first."""
    d = _desc()
    w = B.Weights(*([FAKE] * 7))
    need = lib.e2v2_attn_workspace_bytes(ctypes.byref(d), 100000)
    assert need > 64 << 20
    st = lib.e2v2_attn_forward_noalloc(ctypes.byref(d), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, None, 100000,
                                       FAKE, None)
    assert st == B.E2V2_ERR_CAPACITY and "workspace" in lib.e2v2_last_error().decode()
    assert lib.e2v2_attn_forward_noalloc(None, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, None, 10, FAKE,
                                         None) == B.E2V2_ERR_ARG
    assert lib.e2v2_attn_forward_noalloc(ctypes.byref(d), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, None, -1,
                                         FAKE, None) == B.E2V2_ERR_ARG
    assert lib.e2v2_attn_forward_noalloc(ctypes.byref(d), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, None, 0,
                                         FAKE, None) == B.E2V2_OK
