"""Neighbour reuse and the layer stack on the GPU against the stack oracle:
filtered lists bit-exact, the displacement bit-exact, rebuild steps identical,
stack outputs within the layer's tolerances at every step."""
import numpy as np
import pytest
import torch

from atomistic_attention_amd import workloads as W
from oracle import layer as O
from oracle import stack as OS
from tests._helpers import f32, record, rel_err, rows_from_device, to_storage

pytestmark = pytest.mark.gpu


def _rows_equal(got, want, as_sets=False):
    for i, (a, b) in enumerate(zip(got, want)):
        if not np.array_equal(np.sort(a) if as_sets else a, b):
            raise AssertionError(f"row {i}: gpu {a[:10]} ({a.size}) vs oracle {b[:10]} ({b.size})")


def test_filter_bit_exact_at_5A(gpu_lib):
    """The 8 A, K = 256 list of the 32,768-atom system filtered to 5 A equals the
    brute-force 5 A list row for row (as sets: the builder's rows come in its scan
    order, and the filter keeps the order of the row it filters); in place gives
    the same."""
    wl = W.make_workload("c4")
    pos = f32(wl.pos)
    start, length, idx, _ = gpu_lib.e2v2_build_neighbors(pos, 8.0, 256, want_nnz=False)
    ln5, ix5 = gpu_lib.e2v2_filter_neighbors(pos, 5.0, start, length, idx)
    torch.cuda.synchronize()
    ref = O.neighbors(wl.pos, 5.0)
    got = rows_from_device(start, ln5, ix5)
    _rows_equal(got, ref, as_sets=True)
    rows8 = rows_from_device(start, length, idx)
    for i in range(0, wl.cfg.n, 211):
        keep = np.isin(rows8[i], got[i])
        assert np.array_equal(rows8[i][keep], got[i])            # order kept
    full = ix5.view(wl.cfg.n, 256).cpu().numpy()
    ln_h, l8 = ln5.cpu().numpy(), length.cpu().numpy()
    for i in range(0, wl.cfg.n, 97):
        assert np.all(full[i, ln_h[i]:l8[i]] == -1)
    gpu_lib.e2v2_filter_neighbors(pos, 5.0, start, length, idx, out_len=length, out_idx=idx)
    torch.cuda.synchronize()
    assert torch.equal(length, ln5) and torch.equal(idx.view(-1, 256)[:, :1], ix5.view(-1, 256)[:, :1])
    _rows_equal(rows_from_device(start, length, idx), ref, as_sets=True)


def test_filter_edge_rows(gpu_lib):
    """Invalid and out-of-range entries drop out, order is kept, empty rows stay empty,
    a row longer than one wave chunk compacts across chunks."""
    rng = np.random.default_rng(8)
    n = 300
    pos = rng.uniform(-6, 6, (n, 3)).astype(np.float32).astype(np.float64)
    K = 160
    rows = []
    for i in range(n):
        r = rng.permutation(n)[:rng.integers(0, K)].astype(np.int32)
        r[rng.random(r.size) < 0.1] = -1
        r[rng.random(r.size) < 0.05] = n + 3
        rows.append(r)
    start = np.arange(n, dtype=np.int32) * K
    length = np.array([r.size for r in rows], dtype=np.int32)
    idx = np.full(n * K, -7, dtype=np.int32)
    for i, r in enumerate(rows):
        idx[start[i]:start[i] + r.size] = r
    t = lambda a: torch.from_numpy(a).cuda()
    ln, ix = gpu_lib.e2v2_filter_neighbors(f32(pos), 4.0, t(start), t(length), t(idx))
    torch.cuda.synchronize()
    _rows_equal(rows_from_device(t(start), ln, ix), OS.filter_rows(pos, rows, 4.0))


def test_max_displacement_bit_exact(gpu_lib):
    rng = np.random.default_rng(5)
    ref = rng.uniform(-30, 30, (50000, 3)).astype(np.float32).astype(np.float64)
    pos = (ref + rng.normal(0, 0.05, ref.shape)).astype(np.float32).astype(np.float64)
    got = gpu_lib.e2v2_max_displacement2(f32(pos), f32(ref)).item()
    assert got == OS.max_displacement2(pos, ref)
    pos[123, 1] = np.nan
    assert gpu_lib.e2v2_max_displacement2(f32(pos), f32(ref)).item() == np.inf
    assert gpu_lib.e2v2_max_displacement2(f32(pos[:0]), f32(ref[:0])).item() == 0.0


def _run_gpu(gpu_lib, st):
    dt = torch.bfloat16 if st.base.storage == "bf16" else torch.float32
    descs, weights = [], []
    for wl in st.layers:
        c = wl.cfg
        descs.append(gpu_lib.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, dt))
        weights.append(W.device_arrays(wl)["weights"])
    run = gpu_lib.StackRun(descs, weights, st.cfg.n, st.cfg.max_neighbors)
    h = to_storage(st.h0, dt)
    outs, rebuilt = [], []
    for t, p in enumerate(st.traj):
        o = run.e2v2_stack_forward(f32(p), h)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy().astype(np.float64))
        if run.policy.rebuilt:
            rebuilt.append(t)
    assert run.policy.rebuilds == len(rebuilt)
    return outs, rebuilt


@pytest.mark.parametrize("name,jumps,tol", [("s1", ((4, 11, (0.3, 0.0, 0.0)),), 1e-4),
                                            ("s2", ((2, 5, (0.0, -0.3, 0.0)),), 2e-2)])
def test_stack_matches_oracle(gpu_lib, name, jumps, tol):
    """Every step of the trajectory: the same rebuild steps (the 10-step rule and an
    early one after a 0.3 A jump) and every atom's output within the layer's
    tolerance (fp32 1e-4, bf16 2e-2 of the output RMS)."""
    st = W.make_stack(name, jumps=jumps)
    outs, rebuilt = _run_gpu(gpu_lib, st)
    ref, rb = OS.run_stack(st)
    assert rebuilt == rb
    errs = [rel_err(a, b) for a, b in zip(outs, ref)]
    record(f"stack[{name}]", worst=max(errs), first=errs[0], last=errs[-1])
    assert max(errs) < tol, errs


def test_stack_deterministic_and_reused_lists(gpu_lib):
    """Two runs agree bit for bit; a step without a rebuild takes the kept lists (its
    output equals a single layer chain over the rebuild-time lists)."""
    st = W.make_stack("s1", steps=3)
    a, ra = _run_gpu(gpu_lib, st)
    b, rb = _run_gpu(gpu_lib, st)
    assert ra == rb == [0]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("K", [256, 60])
def test_stack_gradient_matches_oracle(gpu_lib, K):
    """dL/dh and dL/dpos of the four-layer stack (fp32 storage, 256 atoms) after one
    forward call, against the oracle's reverse mode through the same lists; K = 60
    makes the 8 A cap bind, so its list (and the 5 A lists taken from it) are not
    symmetric."""
    import dataclasses
    from oracle import backward as OB
    cfg = dataclasses.replace(W.STACKS["s1"], steps=1, max_neighbors=K)
    st = W.make_stack(cfg)
    descs, weights = [], []
    for wl in st.layers:
        c = wl.cfg
        descs.append(gpu_lib.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, torch.float32))
        weights.append(W.device_arrays(wl)["weights"])
    run = gpu_lib.StackRun(descs, weights, cfg.n, K)
    pos = f32(st.traj[0])
    h = f32(st.h0)
    print(f"stack gradient n={cfg.n} K={K}", flush=True)
    run.e2v2_stack_forward(pos, h)
    g = np.random.default_rng(31).standard_normal(st.h0.shape).astype(np.float32).astype(np.float64)
    gh, gp = run.e2v2_stack_backward(pos, h, f32(g), grad_pos=torch.empty((cfg.n, 3), device="cuda"))
    torch.cuda.synchronize()
    state = OS.StackState([wl.cfg.cutoff for wl in st.layers], K)
    state.rebuild(st.traj[0], 0)
    rp, rh = OB.stack_grad_pos_h(st.traj[0], st.h0, st.layers, state.rows, g)
    eh, ep = rel_err(gh.cpu().numpy(), rh), rel_err(gp.cpu().numpy(), rp)
    record(f"stack_gradient[s1,K={K}]", grad_h=eh, grad_pos=ep)
    assert eh < 1e-4 and ep < 1e-4, (eh, ep)


def test_stack_gradient_bf16_storage(gpu_lib):
    """The four-layer stack at bf16 storage (s2's layers: 5 A, 5 A, 5 A, 8 A, 16 heads,
    l_max = 2), 300 atoms: dL/dh and dL/dpos against the oracle's stack gradient with
    the outputs rounded to bf16 between layers and the rounding passing the gradient
    through (B4).  Each layer's gradient is fp32 arithmetic at bf16 values; the
    inputs of layers 2-4 are the GPU forward's own bf16 outputs, whose 16-bit
    intermediates move about one element in eight by one bf16 step against the
    oracle's rounded outputs, so the bar is the bf16-storage bar of the layer
    output, 2e-2 of the RMS."""
    import dataclasses
    from oracle import backward as OB
    cfg = dataclasses.replace(W.STACKS["s2"], n=300, steps=1)
    st = W.make_stack(cfg)
    descs, weights = [], []
    for wl in st.layers:
        c = wl.cfg
        descs.append(gpu_lib.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, torch.bfloat16))
        weights.append(W.device_arrays(wl)["weights"])
    run = gpu_lib.StackRun(descs, weights, cfg.n, cfg.max_neighbors)
    pos = f32(st.traj[0])
    h = to_storage(st.h0, torch.bfloat16)
    print(f"stack gradient bf16 n={cfg.n}", flush=True)
    run.e2v2_stack_forward(pos, h)
    g = np.random.default_rng(32).standard_normal(st.h0.shape).astype(np.float32).astype(np.float64)
    gh, gp = run.e2v2_stack_backward(pos, h, f32(g), grad_pos=torch.empty((cfg.n, 3), device="cuda"))
    torch.cuda.synchronize()
    state = OS.StackState([wl.cfg.cutoff for wl in st.layers], cfg.max_neighbors)
    state.rebuild(st.traj[0], 0)
    rp, rh = OB.stack_grad_pos_h(st.traj[0], st.h0, st.layers, state.rows, g, round_between=True)
    eh, ep = rel_err(gh.cpu().numpy(), rh), rel_err(gp.cpu().numpy(), rp)
    record(f"stack_gradient_bf16[s2,n={cfg.n}]", grad_h=eh, grad_pos=ep)
    assert eh < 2e-2 and ep < 2e-2, (eh, ep)


def _far_pairs(pos, rows, cutoff):
    """Listed pairs at or beyond ``cutoff`` (fp64 distances of the fp32 positions)."""
    n = 0
    for i, r in enumerate(rows):
        r = np.asarray(r, dtype=np.int64)
        r = r[(r >= 0) & (r < pos.shape[0])]
        if r.size:
            n += int(np.sum(np.linalg.norm(pos[r] - pos[i], axis=1) >= cutoff))
    return n


def _moving_stack(steps):
    """s1 (256 atoms, fp32) with 24 atoms moved by 0.2 A at step 2: below the 0.25 A
    rebuild threshold, so the lists built at step 0 are kept while listed pairs of
    the moved atoms cross 5 A and 8 A."""
    rng = np.random.default_rng(17)
    dirs = rng.standard_normal((24, 3))
    dirs = 0.2 * dirs / np.linalg.norm(dirs, axis=1, keepdims=True)
    jumps = tuple((2, int(a), tuple(v)) for a, v in zip(rng.choice(256, 24, replace=False), dirs))
    return W.make_stack("s1", steps=steps, jumps=jumps)


def test_stack_reused_lists_with_pairs_beyond_the_cutoff(gpu_lib):
    """Tessera article, neighbour reuse: between rebuilds the lists stay as built and
    the layers take distances from the current positions, so listed pairs can lie
    beyond the cutoff.  Their envelope is 0 (FlashSchNet summary section 2.2: the
    cutoff mask): no distance bias, while q.k still counts.  Every step of the
    GPU stack matches the oracle's within 1e-4 of the output RMS."""
    st = _moving_stack(8)
    outs, rebuilt = _run_gpu(gpu_lib, st)
    state = OS.StackState([wl.cfg.cutoff for wl in st.layers], st.cfg.max_neighbors)
    far, errs = 0, []
    for t, p in enumerate(st.traj):
        ref = OS.stack_step(state, p, st.h0, st.layers, t, "fp32")
        if t not in state.rebuilds:
            far += sum(_far_pairs(p, rows, c) for c, rows in state.rows.items())
        errs.append(rel_err(outs[t], ref))
    assert rebuilt == state.rebuilds == [0]
    assert far >= 10, far
    record("stack_far_pairs[s1]", worst=max(errs), far_pairs=far)
    assert max(errs) < 1e-4, errs


def test_stack_gradient_on_reused_lists(gpu_lib):
    """dL/dh and dL/dpos of the four-layer stack after forward steps that reused
    the step-0 lists while atoms moved (pairs beyond 5 A and 8 A among them),
    against the oracle's reverse mode over the rebuild-time lists at the current
    positions."""
    from oracle import backward as OB
    st = _moving_stack(4)
    descs, weights = [], []
    for wl in st.layers:
        c = wl.cfg
        descs.append(gpu_lib.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, torch.float32))
        weights.append(W.device_arrays(wl)["weights"])
    run = gpu_lib.StackRun(descs, weights, st.cfg.n, st.cfg.max_neighbors)
    h = f32(st.h0)
    for p in st.traj:
        run.e2v2_stack_forward(f32(p), h)
    torch.cuda.synchronize()
    assert run.policy.rebuilds == 1
    pos = st.traj[-1]
    g = np.random.default_rng(33).standard_normal(st.h0.shape).astype(np.float32).astype(np.float64)
    gh, gp = run.e2v2_stack_backward(f32(pos), h, f32(g), grad_pos=torch.empty((st.cfg.n, 3), device="cuda"))
    torch.cuda.synchronize()
    state = OS.StackState([wl.cfg.cutoff for wl in st.layers], st.cfg.max_neighbors)
    state.rebuild(st.traj[0], 0)
    assert sum(_far_pairs(pos, rows, c) for c, rows in state.rows.items()) >= 10
    rp, rh = OB.stack_grad_pos_h(pos, st.h0, st.layers, state.rows, g)
    eh, ep = rel_err(gh.cpu().numpy(), rh), rel_err(gp.cpu().numpy(), rp)
    record("stack_gradient_reused[s1]", grad_h=eh, grad_pos=ep)
    assert eh < 1e-4 and ep < 1e-4, (eh, ep)


def test_stack_backward_before_forward_raises(gpu_lib):
    """The state holds no lists before the first forward call: the gradient call
    raises before anything is launched."""
    st = W.make_stack("s1", steps=1)
    descs = [gpu_lib.make_desc(wl.cfg.lmax, wl.cfg.channels, wl.cfg.heads, wl.cfg.n_rbf, wl.cfg.cutoff, torch.float32)
             for wl in st.layers]
    run = gpu_lib.StackRun(descs, [W.device_arrays(wl)["weights"] for wl in st.layers], st.cfg.n, st.cfg.max_neighbors)
    with pytest.raises(gpu_lib.E2V2Error):
        run.e2v2_stack_backward(f32(st.traj[0]), f32(st.h0), f32(np.zeros(st.h0.shape)))
