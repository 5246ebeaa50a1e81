#!/usr/bin/env python3
"""Benchmark of one E2Former-V2 node-centric attention layer forward on one MI355X.

A step is one pass of the whole path over the resident workload: the cell-list
neighbour build (capped, no host synchronisation) followed by the layer forward
(projections, source EAAS coupling, fused streaming attention with the target
coupling, output projection).  The default workload is 32,768 atoms at
0.1 atoms/A^3 with an 8 A cutoff and a K = 256 neighbour cap, l_max = 2,
128 channels, 16 heads, 32 RBFs, bf16 storage with fp32 arithmetic.

Prints one JSON line: pairs/s over the whole step (value), steps/s, per-stage
times, the streaming kernel's achieved algorithmic bandwidth against the HBM
peak (roofline), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--config c4] [--no-cpu-baseline] [--no-stack]

config.stack reports the model level: steps/s of the four-layer stack (three 5 A
layers, one 8 A layer) with neighbour reuse on the same system moving by a random
walk (e2v2_stack_forward).  config.backward reports the feature gradient of one
layer (e2v2_layer_backward) on 32,768 atoms with an uncapped 5 A list and fp32
storage, next to that layer's forward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "atom-neighbour pairs/s & steps/s per attn layer fwd; % HBM peak (1 MI355X)"
HBM_PEAK_GBS = 8000.0
ATTN_SRCS = [os.path.join(ROOT, "atomistic_attention_amd", "csrc", f)
             for f in ("attn_pair.hip", "attn.hip", "attn_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")


def algorithmic_bytes(cfg, nnz: int) -> dict:
    """Bytes the streaming kernel must move: per pair the neighbour's coupled value
    row h'_j and key row k_j, its index and its position -- fp32 rows for fp32
    storage; for bf16 storage fp16 rows, the key travelling with h's odd last
    component in 16-byte pieces (4C bytes) next to h's component pairs; per target
    its query, its position, its row bounds and one output row -- the message m_i
    in fp16 with its node scale for bf16 storage (the target coupling runs in the
    output kernel), the coupled fp32 hhat_i for fp32 storage, which also reads the
    target's D blocks."""
    C, nc = cfg.channels, cfg.n_comp
    nd = sum((2 * l + 1) ** 2 for l in range(1, cfg.lmax + 1))
    if cfg.storage == "bf16":
        per_pair = 2 * (nc & ~1) * C + 4 * C + 4 + 12
    else:
        per_pair = 4 * nc * C + 4 * C + 4 + 12
    if cfg.storage == "bf16":
        per_node = 4 * C + 12 + 8 + 2 * nc * C + 4
    else:
        per_node = 4 * C + 12 + 8 + 4 * nc * C + 4 * nd
    return {"per_pair": per_pair, "per_node": per_node, "total": nnz * per_pair + cfg.n * per_node}


def kernel_hash() -> str:
    """Hash of the streaming kernels' sources (the stored counters are valid for those sources only)."""
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def streaming_kernel(cfg) -> str:
    if cfg.storage == "bf16" and cfg.lmax <= 2:
        return "attn_pair_kernel (two neighbouring targets per wave over the union of their lists; emits m_i)"
    if cfg.storage == "bf16":
        return "attn_kernel (one target per wave; emits the message m_i)"
    return "attn_kernel (one target per wave, + target EAAS)"


def measured_traffic(workload: str):
    """HBM bytes per launch of the streaming kernel from the committed counter runs,
    if they were taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_targets: int | None = None) -> dict:
    """The fp64 oracle on a compact ball of targets around the box centre (all of
    its steps: brute-force neighbours, projections, dense-CG coupling, explicit
    softmax, target coupling, output projection)."""
    from oracle import layer as O
    pos = wl.pos
    r = np.linalg.norm(pos, axis=1)
    T = budget_targets or int(os.environ.get("E2V2_CPU_TARGETS", "2500"))
    tg = np.sort(np.argsort(r, kind="stable")[:T])
    t0 = time.perf_counter()
    res = O.layer_forward_workload(wl, targets=tg)
    dt = time.perf_counter() - t0
    pairs = int(sum(x.size for x in res["rows"]))
    threads = int(os.environ.get("OMP_NUM_THREADS", str(len(os.sched_getaffinity(0)))))
    return {"value": pairs / dt, "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"{T} targets nearest the box centre of the same workload ({pairs} pairs, "
                      f"{res['src'].size} coupled sources), whole layer incl. brute-force neighbours; "
                      f"{dt:.1f} s; the neighbour search uses {threads} OpenMP threads, the numpy "
                      f"tensor products one thread"}


def stack_bench(B, W, torch, steps: int = 60, warmup: int = 10) -> dict:
    """Model-level steps/s of the four-layer stack (5, 5, 5, 8 A) on the 32,768-atom
    system moving by a random walk: every call is one model step with the rebuild
    rule (10 steps, or a move of more than 0.25 A) applied by the library."""
    st = W.make_stack("s4", steps=warmup + steps)
    dt = torch.bfloat16 if st.base.storage == "bf16" else torch.float32
    descs, weights = [], []
    for wl in st.layers:
        c = wl.cfg
        descs.append(B.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, dt))
        weights.append(W.device_arrays(wl)["weights"])
    run = B.StackRun(descs, weights, st.cfg.n, st.cfg.max_neighbors)
    h = W.device_arrays(st.layers[0])["h"]
    traj = [torch.from_numpy(np.ascontiguousarray(p, dtype=np.float32)).cuda() for p in st.traj]
    out = torch.empty(st.h0.shape, dtype=torch.float32, device="cuda")
    for t in range(warmup):
        run.e2v2_stack_forward(traj[t], h, out=out)
    torch.cuda.synchronize()
    r0 = run.policy.rebuilds
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        run.e2v2_stack_forward(traj[t], h, out=out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    c = st.base
    return {"model": f"{len(st.layers)} layers, cutoffs {list(st.cfg.cutoffs)} A, the 8 A list capped at K="
                     f"{st.cfg.max_neighbors} and the 5 A lists filtered from it; l_max={c.lmax}, C={c.channels}, "
                     f"{c.heads} heads, {c.n_rbf} RBFs, {c.storage} storage",
            "atoms": st.cfg.n, "steps": steps, "ms_per_step": ms, "steps_per_s": 1e3 / ms,
            "rebuilds": int(run.policy.rebuilds - r0),
            "rebuild_rule": "every 10 steps, or when an atom moved more than 0.25 A since the last rebuild",
            "trajectory": f"random walk, N(0, {st.cfg.sigma}^2) A per coordinate and step, synthetic"}


def backward_bench(B, W, torch, steps: int = 20, warmup: int = 3, name: str = "g4") -> dict:
    """Gradient of one layer (e2v2_layer_backward: the forward's projections and
    source coupling, then the adjoint chain; dL/dh, and dL/dh with dL/dpos) on the 32,768-atom
    system with an uncapped 5 A list and fp32 storage, next to the forward of the
    same layer.  Both timed on resident inputs and lists built beforehand, in the
    list's spatial order."""
    wl = W.make_workload(name)
    c = wl.cfg
    d = W.device_arrays(wl)
    dev = d["pos"].device
    desc = B.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, torch.float32)
    order = torch.empty(c.n, dtype=torch.int32, device=dev)
    s, ln, ix, nnz = B.e2v2_build_neighbors(d["pos"], c.cutoff, 0, order_out=order)
    g = torch.from_numpy(np.random.default_rng(11).standard_normal(wl.h.shape).astype(np.float32)).to(dev)
    gh = torch.empty_like(g)
    out = torch.empty_like(g)
    bws = torch.empty(B.backward_workspace_bytes(desc, c.n, ix.numel()), dtype=torch.uint8, device=dev)
    fws = torch.empty(B.attn_workspace_bytes(desc, c.n), dtype=torch.uint8, device=dev)

    gp = torch.empty((c.n, 3), dtype=torch.float32, device=dev)

    def bwd():
        B.e2v2_layer_backward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, g, grad_h=gh, workspace=bws,
                              target_order=order, symmetric=True)

    def bwd_pos():
        B.e2v2_layer_backward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, g, grad_h=gh, workspace=bws,
                              target_order=order, grad_pos=gp, symmetric=True)

    def fwd():
        B.e2v2_attn_forward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, out=out, workspace=fws,
                            target_order=order)

    def train_step():
        # the forward on the gradient's workspace, then both gradients reusing its q, k, v, h'
        B.e2v2_attn_forward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, out=out, workspace=bws,
                            target_order=order)
        B.e2v2_layer_backward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, g, grad_h=gh, workspace=bws,
                              target_order=order, grad_pos=gp, symmetric=True, reuse_forward=True)

    res = {}
    for key, fn in (("backward", bwd), ("backward_pos", bwd_pos), ("forward", fwd), ("train", train_step)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res[key] = (time.perf_counter() - t0) * 1e3 / steps
    # the four-layer stack in fp32 storage on the same system: one model step forward,
    # then dL/dh and dL/dpos of the whole model (the forces for E = sum(g * out))
    import dataclasses
    sc = dataclasses.replace(W.STACKS["s4"], base=name, steps=1)
    stk = W.make_stack(sc)
    sdescs, sweights = [], []
    for wl in stk.layers:
        lc = wl.cfg
        sdescs.append(B.make_desc(lc.lmax, lc.channels, lc.heads, lc.n_rbf, lc.cutoff, torch.float32))
        sweights.append(W.device_arrays(wl)["weights"])
    run = B.StackRun(sdescs, sweights, sc.n, sc.max_neighbors, rebuild_every=1 << 30, max_displacement=1e9)
    spos = torch.from_numpy(np.ascontiguousarray(stk.traj[0], dtype=np.float32)).to(dev)
    sh = torch.from_numpy(np.ascontiguousarray(stk.h0, dtype=np.float32)).to(dev)
    sout = torch.empty(stk.h0.shape, dtype=torch.float32, device=dev)
    sgh = torch.empty_like(sout)
    sgp = torch.empty((sc.n, 3), dtype=torch.float32, device=dev)
    run.e2v2_stack_forward(spos, sh, out=sout)                      # builds the lists once
    for key, fn in (("stack_forward", lambda: run.e2v2_stack_forward(spos, sh, out=sout)),
                    ("stack_gradients", lambda: run.e2v2_stack_backward(spos, sh, g, grad_h=sgh, grad_pos=sgp))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        res[key] = (time.perf_counter() - t0) * 1e3 / 5
    nnz = int(nnz)
    C, nc, H = c.channels, c.n_comp, c.heads
    # attention adjoint, algorithmic bytes: target pass per pair k_j, h'_j, position,
    # index; source pass per pair q_i, dm_i, position, index and (mx, rz, dd) of the
    # 16 heads; per node the own rows in and the gradients out
    per_pair = 2 * (4 * C + 4 * nc * C + 16 + 4) + 3 * 4 * H
    per_node = 2 * (4 * C + 4 * nc * C + 16 + 8) + 4 * C + 3 * 4 * H + 4 * nc * C + 4 * C
    return {"workload": f"{name}: {c.n} atoms, {c.geometry} at {c.density} atoms/A^3, cutoff {c.cutoff} A "
                        f"uncapped (symmetric list), l_max={c.lmax}, C={C}, {H} heads, {c.n_rbf} RBFs, "
                        f"fp32 storage",
            "what": "dL/dh for L = sum(g * out), g fixed (ms_backward); dL/dh and dL/dpos together "
                    "(ms_backward_with_positions); weights and the neighbour list held fixed; the uncapped list "
                    "is symmetric and serves as its own transpose; ms_forward_then_gradients: the forward, then "
                    "dL/dh and dL/dpos reusing the forward's q, k, v, h' (one training step of the layer)",
            "nnz": nnz, "steps": steps, "ms_backward": res["backward"],
            "ms_backward_with_positions": res["backward_pos"], "ms_forward_same_layer": res["forward"],
            "ms_forward_then_gradients": res["train"],
            "stack_fp32": {"model": "four layers (5, 5, 5, 8 A; the 8 A list capped at K=256, the 5 A lists "
                                    "filtered from it), fp32 storage, same system, lists reused",
                           "ms_model_step_forward": res["stack_forward"],
                           "ms_gradients_dh_dpos": res["stack_gradients"]},
            "pairs_per_s_backward": nnz / (res["backward"] * 1e-3),
            "pairs_per_s_backward_with_positions": nnz / (res["backward_pos"] * 1e-3),
            "attention_adjoint_algorithmic_bytes": per_pair * nnz + per_node * c.n}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the four-layer stack measurement")
    ap.add_argument("--stack-only", action="store_true",
                    help="run only the four-layer stack measurement and print its record (for profiling)")
    ap.add_argument("--no-backward", action="store_true", help="skip the feature-gradient measurement")
    ap.add_argument("--backward-only", action="store_true",
                    help="run only the feature-gradient measurement and print its record (for profiling)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for hardware-counter runs: 3 layer forwards, then 3 plain device copies of 1 GiB "
                         "(the copies calibrate the counters' byte units); prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this layer has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from atomistic_attention_amd import binding as B
    from atomistic_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.load()
    if args.stack_only:
        print(json.dumps({"stack": stack_bench(B, W, torch)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": backward_bench(B, W, torch)}), flush=True)
        return
    wl = W.make_workload(args.config)
    cfg = wl.cfg
    d = W.device_arrays(wl)
    dev = d["pos"].device
    desc = B.make_desc(cfg.lmax, cfg.channels, cfg.heads, cfg.n_rbf, cfg.cutoff, d["dtype"])
    N, K = cfg.n, cfg.max_neighbors
    # resident buffers
    start = torch.empty(N, dtype=torch.int32, device=dev)
    length = torch.empty(N, dtype=torch.int32, device=dev)
    order = torch.empty(N, dtype=torch.int32, device=dev)
    s0, l0, i0, nnz = B.e2v2_build_neighbors(d["pos"], cfg.cutoff, K)
    cap = i0.numel()
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    out = torch.empty(wl.h.shape, dtype=torch.float32, device=dev)
    nws = torch.empty(B.load().e2v2_build_neighbors_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    aws = torch.empty(B.attn_workspace_bytes(desc, N), dtype=torch.uint8, device=dev)
    lib = B.load()
    stream = torch.cuda.current_stream()
    import ctypes

    def build():
        if K > 0:
            st = lib.e2v2_build_neighbors(B._ptr(d["pos"]), N, float(cfg.cutoff), K, B._ptr(start), B._ptr(length),
                                          B._ptr(idx), cap, None, B._ptr(order), B._ptr(nws), nws.numel(),
                                          B._stream())
            B._check(st)
        else:   # CSR needs the nnz read-back (one host synchronisation)
            n64 = ctypes.c_int64(0)
            st = lib.e2v2_build_neighbors(B._ptr(d["pos"]), N, float(cfg.cutoff), 0, B._ptr(start), B._ptr(length),
                                          B._ptr(idx), cap, ctypes.byref(n64), B._ptr(order), B._ptr(nws),
                                          nws.numel(), B._stream())
            B._check(st)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for row in events:
        for e in row:
            e.record(stream)          # creates the underlying events
    torch.cuda.synchronize()

    def step(ev=None):
        """One step in stage order on one stream (events mark the stage boundaries)."""
        if ev is not None:
            ev[0].record(stream)
        build()
        B.e2v2_attn_forward(desc, d["pos"], d["h"], d["weights"], start, length, idx, out=out, workspace=aws,
                            taps={"events": ev[1:]} if ev is not None else None, target_order=order)

    # The timed step: the projections and source coupling need no neighbour list,
    # so they run on a second stream while the list is built, and the streaming
    # attention + output stage joins both.  The fork waits for the previous step,
    # whose attention still reads the workspace.
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def step_overlapped():
        fork.record(stream)
        side.wait_event(fork)
        B.e2v2_attn_prepare(desc, d["pos"], d["h"], d["weights"], aws, stream=side)
        join.record(side)
        build()
        stream.wait_event(join)
        B.e2v2_attn_aggregate(desc, d["weights"], start, length, idx, out, aws, stream=stream, target_order=order)

    if args.traffic_probe:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(f"traffic probe: 5 steps of {cfg.name} (1 attention launch each), 3 copies of {x.numel() * 4} bytes",
              flush=True)
        return

    for _ in range(args.warmup):
        step_overlapped()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step_overlapped()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # Stage times (and the streaming kernel's launch time for the roofline) from the
    # same number of steps run in stage order on one stream, outside the timed region.
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    stages = np.array([[events[k][a].elapsed_time(events[k][a + 1]) for a in range(5)] for k in range(args.steps)])
    mean = stages.mean(axis=0)          # ms per stage between consecutive events
    serial_ms = float(stages.sum(axis=1).mean())
    nnz = int(length.sum().item())
    ab = algorithmic_bytes(cfg, nnz)
    t_attn = mean[3] * 1e-3
    achieved = ab["total"] / t_attn / 1e9
    traffic = measured_traffic(cfg.name)
    layer_ms = float(mean[1:].sum())
    C, nc, s = cfg.channels, cfg.n_comp, (2 if cfg.storage == "bf16" else 4)
    nd = sum((2 * l + 1) ** 2 for l in range(1, cfg.lmax + 1))
    if cfg.storage == "bf16":
        # fused projections + source EAAS: h and positions in; q, the key + tail rows,
        # h's component pairs, D blocks, pos4 out
        front = N * nc * C * 2 + N * 12 + N * C * 4 + N * C * 4 + N * (nc & ~1) * C * 2 + N * (4 * nd + 16)
        stage_names = ("neighbours", "projections+source_eaas", None, "attention", "target_eaas+output_projection")
        front += N * (4 * nd + 16)          # the back end reads the D blocks and pos4 again
    else:
        front = (N * nc * C * s + N * C * 8 + N * nc * C * 4                          # projections
                 + N * nc * C * 4 + N * 12 + N * nc * C * s + N * (4 * nd + 16))    # source EAAS
        stage_names = ("neighbours", "projections", "source_eaas", "attention", "output_projection")
    back = N * (2 * nc * C + 4) + N * nc * C * 4 if cfg.storage == "bf16" else 2 * N * nc * C * 4
    layer_bytes = (front
                   + ab["total"]                                          # streaming attention + target EAAS
                   + back)                                                # (target EAAS +) output projection
    stage_ms = {}
    for name, v in zip(stage_names, mean):
        if name is None:
            stage_ms[prev] += float(v)      # the two events of a fused stage are recorded back to back
        else:
            stage_ms[name] = float(v)
            prev = name

    rec = {
        "metric": METRIC,
        "value": nnz / (ms_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {N} atoms, {cfg.geometry} at {cfg.density} atoms/A^3, cutoff {cfg.cutoff} A, "
                        f"cap K={K}, l_max={cfg.lmax}, C={cfg.channels}, {cfg.heads} heads, {cfg.n_rbf} RBFs, "
                        f"{cfg.storage} storage, fp32 arithmetic",
            "nnz": nnz,
            "steps_per_s": 1e3 / ms_step,
            "stage_ms": stage_ms,
            "stages_in_order_ms_per_step": serial_ms,
            "overlap": "projections + source coupling on a second stream during the neighbour build",
            "layer_ms_excl_neighbours": layer_ms,
            "layer_pairs_per_s_excl_neighbours": nnz / (layer_ms * 1e-3),
            "layer_hbm_frac_excl_neighbours": layer_bytes / (layer_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        },
        "roofline": {
            "kernel": streaming_kernel(cfg),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["total"],
            "bytes_per_pair": ab["per_pair"],
            "bytes_per_target": ab["per_node"],
            "avg_launch_ms": float(mean[3]),
            "note": "achieved counts every (target, neighbour) pair's row (algorithmic bytes); rows shared by "
                    "the two targets of a wave are loaded once, and rows shared by nearby targets are served "
                    "from L2/MALL, so HBM traffic is a small part of it (see traffic) and frac can exceed 1",
        },
        "cpu_baseline": None,
    }
    if not args.no_stack:
        rec["config"]["stack"] = stack_bench(B, W, torch)
    if not args.no_backward:
        rec["config"]["backward"] = backward_bench(B, W, torch)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
