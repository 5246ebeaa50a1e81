#!/usr/bin/env python3
"""Benchmark of one E2Former-V2 node-centric attention layer forward on one MI355X.

A step is one pass of the whole path over the resident workload: the cell-list
neighbour build (capped, no host synchronisation) followed by the layer forward
(projections, source EAAS coupling, fused streaming attention with the target
coupling, output projection).  The default workload is 32,768 atoms at
0.1 atoms/A^3 with an 8 A cutoff and a K = 256 neighbour cap, l_max = 2,
128 channels, 16 heads, 32 RBFs, bf16 storage with fp32 arithmetic.

Prints one JSON line: pairs/s over the whole step (value), steps/s, per-stage
times, the streaming kernel against the resource that binds it (roofline: fp32
ALU on algorithmic flops; beside it the VALU issue share, DRAM and L2-miss bytes
from committed counter runs, and the algorithmic byte count against the HBM
peak), records of the other configurations (config.per_config, with the
clustered system's load balance), and the fp64 CPU oracle timed on a bounded
sample of the same workload on this host (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--config c4] [--no-cpu-baseline] [--no-stack]
                    [--no-backward] [--no-per-config]

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
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published (counts packed fp32: two values per lane)
CLOCK_GHZ = 2.4
SIMDS = 256 * 4                # 256 CUs x 4 SIMDs
ATTN_SRCS = [os.path.join(ROOT, "atomistic_attention_amd", "csrc", f)
             for f in ("attn_quad.hip", "attn_pair.hip", "attn.hip", "attn_common.h")]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_counters.json")
PER_CONFIG = ("c1", "c2", "c3", "c3b", "c5")


def algorithmic(cfg, nnz: int) -> dict:
    """What the streaming step moves and computes by the method's own count: per
    (target, neighbour) pair the neighbour's
    coupled value row h'_j in the storage dtype, its fp32 key row, its index and its
    position (n_c C s + 4 C + 16 bytes) and 2 (C + R H + n_c C) flops (logit, bias,
    accumulation); per target its fp32 query and fp32 message plus position and row
    bounds (4 C + 4 n_c C + 20 bytes).  Rows that nearby targets share are counted
    once per pair, so this is a gather-byte count: over the launch time it can
    exceed the HBM peak when the shared rows come from the caches."""
    C, nc, H, R = cfg.channels, cfg.n_comp, cfg.heads, cfg.n_rbf
    s = 2 if cfg.storage == "bf16" else 4
    per_pair = nc * C * s + 4 * C + 16
    per_node = 4 * C + 4 * nc * C + 20
    flops_pair = 2 * (C + R * H + nc * C)
    return {"bytes_per_pair": per_pair, "bytes_per_node": per_node,
            "bytes": nnz * per_pair + cfg.n * per_node, "flops_per_pair": flops_pair, "flops": nnz * flops_pair}


def kernel_hash() -> str:
    """Hash of the streaming kernels' sources (stored counters hold for those sources only)."""
    h = hashlib.sha256()
    for f in ATTN_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def streaming_kernel(cfg) -> str:
    if cfg.storage == "bf16" and cfg.lmax <= 2 and cfg.heads == 16 and cfg.channels == 128:
        return ("attn_quad_kernel (four neighbouring targets per wave over the union of their lists, "
                "logits, bias and weighted sums on the matrix cores; emits m_i)")
    if cfg.storage == "bf16" and cfg.lmax <= 2:
        return "attn_pair_kernel (two neighbouring targets per wave over the union of their lists; emits m_i)"
    if cfg.storage == "bf16":
        return "attn_kernel (one target per wave; emits the message m_i)"
    return "k_attn_f32 (one target per wave, + target EAAS)"


def stored_counters(workload: str):
    """Hardware counters of the streaming kernel for this workload from the committed
    rocprofv3 runs (profiles/), if they were taken on the current kernel sources."""
    try:
        rec = json.load(open(COUNTERS_FILE)).get(workload)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("kernel_sha") != kernel_hash():
        return None
    return rec


def roofline(cfg, nnz: int, t_ms: float) -> dict:
    """The streaming kernel against the resource that binds it.  Its algorithmic
    bytes exceed the HBM peak over its launch time (shared rows are served by L2
    and the MALL), and the counters show the SIMDs' instruction issue, not DRAM, as
    the limit, so the line is the fp32 ALU roofline: algorithmic flops over the
    measured launch time against the fp32 vector peak.  Next to it: the fraction of
    the SIMDs' VALU issue slots used (SQ_INSTS_VALU, 4 cycles per wave64
    instruction), the DRAM bytes (TCC_EA0 request counters) and the L2-miss bytes
    (FETCH_SIZE + WRITE_SIZE), each calibrated by a 1 GiB copy, and the algorithmic
    byte count as a fraction of the HBM peak."""
    a = algorithmic(cfg, nnz)
    t = t_ms * 1e-3
    tf = a["flops"] / t / 1e12
    rec = {"kernel": streaming_kernel(cfg), "bound": "alu", "achieved": tf, "peak": FP32_VALU_PEAK_TFLOPS,
           "unit": "TFLOP/s", "frac": tf / FP32_VALU_PEAK_TFLOPS, "traffic": None,
           "avg_launch_ms": t_ms, "algorithmic_flops_per_launch": a["flops"], "flops_per_pair": a["flops_per_pair"],
           "algorithmic_bytes_per_launch": a["bytes"], "bytes_per_pair": a["bytes_per_pair"],
           "bytes_per_target": a["bytes_per_node"],
           "algorithmic_frac": a["bytes"] / t / (HBM_PEAK_GBS * 1e9),
           "algorithmic_frac_note": "algorithmic gather bytes per launch / launch time / 8 TB/s: every "
                                    "(target, neighbour) pair's rows counted, so it exceeds 1 when rows shared by "
                                    "nearby targets come from L2 and the MALL; not an HBM measurement"}
    ctr = stored_counters(cfg.name)
    if ctr:
        cyc = ctr["launch_ms"] * 1e-3 * CLOCK_GHZ * 1e9
        rec["traffic"] = ctr["fetch_bytes"] + ctr["write_bytes"]
        rec["traffic_what"] = ("L2-miss bytes per launch: FETCH_SIZE + WRITE_SIZE calibrated by a 1 GiB copy; "
                               "reads served by the MALL count too")
        rec["dram_bytes"] = ctr["dram_read_bytes"] + ctr["dram_write_bytes"]
        rec["dram_frac"] = rec["dram_bytes"] / (ctr["launch_ms"] * 1e-3) / (HBM_PEAK_GBS * 1e9)
        rec["valu_issue_frac"] = ctr["valu_insts"] * 4 / (SIMDS * cyc)
        rec["counters"] = {k: ctr[k] for k in ("kernel_sha", "launch_ms", "valu_insts", "fetch_bytes", "write_bytes",
                                                 "dram_read_bytes", "dram_write_bytes")}
    return rec


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_targets: int | None = None) -> dict:
    """The fp64 oracle on a compact ball of targets around the box centre, every step
    of it: O1 brute-force neighbours (C, OpenMP), then O2-O8 (projections, dense-CG
    couplings, explicit softmax, output projection; numpy, its BLAS calls threaded)."""
    from oracle import layer as O
    pos = wl.pos
    c = wl.cfg
    r = np.linalg.norm(pos, axis=1)
    T = budget_targets or int(os.environ.get("E2V2_CPU_TARGETS", "2500"))
    tg = np.sort(np.argsort(r, kind="stable")[:T])
    t0 = time.perf_counter()
    rows = O.neighbors(pos, c.cutoff, c.max_neighbors, targets=tg)
    t1 = time.perf_counter()
    res = O.layer_forward_workload(wl, targets=tg, rows=rows)
    t2 = time.perf_counter()
    pairs = int(sum(x.size for x in rows))
    cores = len(os.sched_getaffinity(0))
    t_layer = t2 - t1
    return {"value": pairs / t_layer, "unit": "pairs/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{T} targets nearest the box centre of the same workload ({pairs} pairs, "
                      f"{res['src'].size} coupled sources)",
            "o1_neighbours_s": t1 - t0, "o2_o8_layer_s": t_layer,
            "sample_steps_per_s": 1.0 / t_layer,
            "full_step_s_estimate": t_layer * c.n / T,
            "threads": f"O1 uses {cores} OpenMP threads; O2-O8 run in numpy with its BLAS threads"}


def per_config(B, W, torch, name: str, steps: int = 20) -> dict:
    """One configuration's layer on its own: the list and the Hilbert processing
    order built once beforehand, then the layer (prepare + aggregate) and its
    streaming kernel timed with HIP events; nnz, ms, pairs/s, steps/s and the
    roofline."""
    wl = W.make_workload(name)
    c = wl.cfg
    d = W.device_arrays(wl)
    dev = d["pos"].device
    desc = B.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, d["dtype"])
    s, ln, ix, nnz = B.e2v2_build_neighbors(d["pos"], c.cutoff, c.max_neighbors)
    order = B.e2v2_target_order(d["pos"])
    aws = torch.empty(B.attn_workspace_bytes(desc, c.n), dtype=torch.uint8, device=dev)
    out = torch.empty(wl.h.shape, dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for e in ev:
        e.record()
    stream = torch.cuda.current_stream()
    nb_ws = torch.empty(B.load().e2v2_build_neighbors_workspace_bytes(c.n, c.max_neighbors), dtype=torch.uint8,
                        device=dev)
    t_layer, t_attn, t_nbr = [], [], []
    for k in range(steps + 3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        B.e2v2_build_neighbors(d["pos"], c.cutoff, c.max_neighbors, workspace=nb_ws, want_nnz=False)
        e1.record(stream)
        B.e2v2_attn_forward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, out=out, workspace=aws,
                            taps={"events": ev}, target_order=order)
        torch.cuda.synchronize()
        if k >= 3:
            t_nbr.append(e0.elapsed_time(e1))
            t_layer.append(ev[0].elapsed_time(ev[4]))
            t_attn.append(ev[2].elapsed_time(ev[3]))
    ms_layer, ms_attn, ms_nbr = (float(np.median(x)) for x in (t_layer, t_attn, t_nbr))
    rl = roofline(c, int(nnz), ms_attn)
    rec = {"workload": f"{name}: {c.n} atoms, {c.geometry} at {c.density} atoms/A^3, cutoff {c.cutoff} A, "
                       f"K={c.max_neighbors or 'none'}, l_max={c.lmax}, C={c.channels}, {c.heads} heads, "
                       f"{c.n_rbf} RBFs, {c.storage} storage",
           "nnz": int(nnz), "steps": steps, "ms_layer": ms_layer, "ms_attention": ms_attn, "ms_neighbours": ms_nbr,
           "pairs_per_s": nnz / (ms_layer * 1e-3), "steps_per_s": 1e3 / ms_layer,
           "steps_per_s_with_neighbours": 1e3 / (ms_layer + ms_nbr),
           "attention_algorithmic_frac": rl["algorithmic_frac"], "attention_alu_frac": rl["frac"],
           "attention_tflops": rl["achieved"]}
    for k in ("traffic", "dram_bytes", "dram_frac", "valu_issue_frac"):
        if k in rl and rl[k] is not None:
            rec["attention_" + k] = rl[k]
    if name == "c5":
        rec["load_balance"] = load_balance(B, W, torch, wl, d, desc, s, ln, ix, order)
    return rec


def xcd_slot_ranges(n: int, per_block: int = 16):
    """The contiguous runs of processing slots that the streaming kernel's XCD-aware
    workgroup mapping gives each of the 8 XCDs (blocks of 4 waves, 4 targets a wave)."""
    nb = (n + per_block - 1) // per_block
    out, b0 = [], 0
    for x in range(8):
        cnt = (nb >> 3) + (1 if x < (nb & 7) else 0)
        out.append((min(n, per_block * b0), min(n, per_block * (b0 + cnt))))
        b0 += cnt
    return out


def load_balance(B, W, torch, wl, d, desc, s, ln, ix, order, reps: int = 10) -> dict:
    """The clustered system's imbalance, two ways.  Static: the share of list entries
    each XCD's run of processing slots holds (max over mean; the XCDs run their runs
    side by side).  Measured: the aggregation run on the targets of the dense blocks
    only and of the sparse blocks only, against all targets, each timed with HIP
    events; the kept targets go four by four (consecutive in the processing order, as
    the kernel groups them) to wave slots spread evenly over the launch, the other
    slots are -1 and their waves exit at once.  Per-target time and row length show
    what a dense region costs; the Tessera article reports 13-33 % slower steps for
    its dense capsid than for its salt solution of similar size."""
    c = wl.cfg
    dev = d["pos"].device
    dense = W.dense_block_mask(wl)
    o = order.cpu().numpy()
    lens = ln.cpu().numpy().astype(np.int64)
    runs = [int(lens[o[a:b]].sum()) for a, b in xcd_slot_ranges(c.n)]
    dense_runs = [float(dense[o[a:b]].mean()) for a, b in xcd_slot_ranges(c.n)]
    aws = torch.empty(B.attn_workspace_bytes(desc, c.n), dtype=torch.uint8, device=dev)
    out = torch.empty(wl.h.shape, dtype=torch.float32, device=dev)
    B.e2v2_attn_prepare(desc, d["pos"], d["h"], d["weights"], aws)
    res = {"xcd_entries": runs, "xcd_dense_fraction": dense_runs,
           "xcd_max_over_mean": max(runs) / (sum(runs) / len(runs))}
    for key, sel in (("all", np.ones(c.n, bool)), ("dense", dense), ("sparse", ~dense)):
        kept = o[sel[o]].astype(np.int32)                     # kept targets in processing order
        nquad_slots, nquads = c.n // 4, (kept.size + 3) // 4
        oo = np.full(c.n, -1, np.int32)
        w = np.arange(nquads, dtype=np.int64)
        if nquads <= nquad_slots:                             # spread; else packed (n not a multiple of 4)
            w = (w * nquad_slots) // nquads
        for i in range(4):
            part = kept[i::4]
            oo[4 * w[: part.size] + i] = part
        ot = torch.from_numpy(oo).to(dev)
        times = []
        for k in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.e2v2_attn_aggregate(desc, d["weights"], s, ln, ix, out, aws, target_order=ot)
            e1.record()
            torch.cuda.synchronize()
            if k >= 2:
                times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        nt = int(sel.sum())
        res[key] = {"targets": nt, "pairs": int(lens[sel].sum()), "mean_row": float(lens[sel].mean()),
                    "ms": ms, "us_per_target": ms * 1e3 / nt, "ns_per_pair": ms * 1e6 / max(int(lens[sel].sum()), 1)}
    res["dense_vs_sparse_per_target"] = res["dense"]["us_per_target"] / res["sparse"]["us_per_target"]
    res["what"] = ("aggregation (attention + target coupling + output projection) over the dense blocks' targets "
                   "only, the sparse blocks' only, and all, with the kept target quads spread evenly over the "
                   "wave slots; xcd_entries: list entries in each XCD's run of the processing order")
    return res


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
    s, ln, ix, nnz = B.e2v2_build_neighbors(d["pos"], c.cutoff, 0)
    order = B.e2v2_target_order(d["pos"])
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
    # forces at the benched configuration: the 32,768-atom, 8 A, K = 256 layer with
    # bf16 storage (gradient in fp32 arithmetic at the bf16 inputs and weights; the
    # capped list is not symmetric, so the call builds its transpose)
    wb = W.make_workload("c4")
    cb = wb.cfg
    db = W.device_arrays(wb)
    descb = B.make_desc(cb.lmax, cb.channels, cb.heads, cb.n_rbf, cb.cutoff, db["dtype"])
    sb_, lb_, ib_, nnzb = B.e2v2_build_neighbors(db["pos"], cb.cutoff, cb.max_neighbors)
    ob = B.e2v2_target_order(db["pos"])
    gb = torch.from_numpy(np.random.default_rng(12).standard_normal(wb.h.shape).astype(np.float32)).to(dev)
    ghb, gpb = torch.empty_like(gb), torch.empty((cb.n, 3), dtype=torch.float32, device=dev)
    outb = torch.empty_like(gb)
    bwsb = torch.empty(B.backward_workspace_bytes(descb, cb.n, ib_.numel()), dtype=torch.uint8, device=dev)
    fwsb = torch.empty(B.attn_workspace_bytes(descb, cb.n), dtype=torch.uint8, device=dev)
    for key, fn in (("c4_gradients", lambda: B.e2v2_layer_backward(descb, db["pos"], db["h"], db["weights"], sb_, lb_,
                                                                    ib_, gb, grad_h=ghb, workspace=bwsb,
                                                                    target_order=ob, grad_pos=gpb)),
                    ("c4_forward", lambda: B.e2v2_attn_forward(descb, db["pos"], db["h"], db["weights"], sb_, lb_, ib_,
                                                               out=outb, workspace=fwsb, target_order=ob))):
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
            "benched_config_bf16": {"workload": f"c4: {cb.n} atoms, cutoff {cb.cutoff} A, cap K={cb.max_neighbors}, "
                                                f"bf16 storage", "nnz": int(nnzb),
                                    "what": "dL/dh and dL/dpos (the forces for E = sum(g * out)) in fp32 arithmetic "
                                            "at the bf16 inputs and weights, transposed list built in the call",
                                    "ms_gradients_dh_dpos": res["c4_gradients"], "ms_forward": res["c4_forward"]},
            "pairs_per_s_backward": nnz / (res["backward"] * 1e-3),
            "pairs_per_s_backward_with_positions": nnz / (res["backward_pos"] * 1e-3),
            "attention_adjoint_algorithmic_bytes": per_pair * nnz + per_node * c.n}


def edge_bench(B, W, torch, steps: int = 10, warmup: int = 2, name: str = "g4") -> dict:
    """The exact edge-equivalent form (e2v2_edge_forward: per-edge tensor products with
    solid harmonics of r_j - r_i, evaluated node by node through 6j recoupling) on the
    32,768-atom system with an uncapped 5 A list, fp32 storage, next to the layer's
    forward on the same system and list; both timed with HIP events."""
    from atomistic_attention_amd.workloads import num_paths
    wl = W.make_workload(name)
    c = wl.cfg
    d = W.device_arrays(wl)
    dev = d["pos"].device
    desc = B.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, torch.float32)
    s, ln, ix, nnz = B.e2v2_build_neighbors(d["pos"], c.cutoff, 0)
    order = B.e2v2_target_order(d["pos"])
    w_e = torch.from_numpy(np.random.default_rng(9).standard_normal((num_paths(c.lmax), c.channels))
                           .astype(np.float32)).to(dev)
    out = torch.empty(wl.h.shape, dtype=torch.float32, device=dev)
    ews = torch.empty(B.edge_workspace_bytes(desc, c.n), dtype=torch.uint8, device=dev)
    aws = torch.empty(B.attn_workspace_bytes(desc, c.n), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms_edge = timed(lambda: B.e2v2_edge_forward(desc, d["pos"], d["h"], d["weights"], w_e, s, ln, ix, out=out,
                                                workspace=ews, target_order=order))
    ms_layer = timed(lambda: B.e2v2_attn_forward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, out=out,
                                                 workspace=aws, target_order=order))
    ngp = {0: 20, 1: 20, 2: 60}[c.lmax]
    return {"workload": f"{name}: {c.n} atoms, {c.geometry} at {c.density} atoms/A^3, cutoff {c.cutoff} A uncapped, "
                        f"l_max={c.lmax}, C={c.channels}, {c.heads} heads, {c.n_rbf} RBFs, fp32 storage",
            "nnz": int(nnz), "steps": steps, "ms_edge_forward": ms_edge, "ms_layer_forward_same_system": ms_layer,
            "pairs_per_s": nnz / (ms_edge * 1e-3), "steps_per_s": 1e3 / ms_edge,
            "source_row_bytes": ngp * c.channels * 4,
            "what": "out = W_O sum_j alpha_ij sum_p w_e[p] (v_j (x) S((r_j - r_i) / r_c))_p evaluated node by node: "
                    "sources coupled with S of their own position (58 components per channel, padded to 60), "
                    "the stream sums alpha-weighted rows, targets recouple with S of their own position"}


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
    ap.add_argument("--no-per-config", action="store_true", help="skip the records of the other configurations")
    ap.add_argument("--no-edge", action="store_true", help="skip the edge-form measurement")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for hardware-counter runs: 5 layer steps of --config, then 3 plain device copies of "
                         "1 GiB (the copies calibrate the counters' byte units); prints no JSON")
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

    # The timed step: the projections and source coupling (which need no neighbour
    # list) on a second stream while the list and the targets' Hilbert processing
    # order are built; the streaming attention + output stage joins both.  The fork
    # waits for the previous step, whose attention still reads the workspace and
    # the order.  The one-stream step in stage order is timed beside it.
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

    def timed(fn, steps):
        """HIP events on the main stream around the whole loop of `steps` calls."""
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    for _ in range(args.warmup):
        step()
    one_stream_ms = timed(step, args.steps)
    for _ in range(args.warmup):
        step_overlapped()
    ms_step = timed(step_overlapped, args.steps)

    # Stage times (and the streaming kernel's launch time for the roofline) from
    # events at the stage boundaries of the same number of steps, outside the timed
    # region.
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    stages = np.array([[events[k][a].elapsed_time(events[k][a + 1]) for a in range(5)] for k in range(args.steps)])
    mean = stages.mean(axis=0)          # ms per stage between consecutive events
    nnz = int(length.sum().item())
    t_attn_ms = float(mean[3])
    layer_ms = float(mean[1:].sum())
    if cfg.storage == "bf16":
        stage_names = ("neighbours+order", "projections+source_eaas", None, "attention",
                       "target_eaas+output_projection")
    else:
        stage_names = ("neighbours+order", "projections", "source_eaas", "attention", "output_projection")
    stage_ms = {}
    for name, v in zip(stage_names, mean):
        if name is None:
            stage_ms[prev] += float(v)      # the two events of a fused stage are recorded back to back
        else:
            stage_ms[name] = float(v)
            prev = name
    a = algorithmic(cfg, nnz)
    # the whole layer (A2-A6) by the same per-unit count: the streaming bytes above
    # plus the node kernels' (A3 reads h and writes h' in the storage dtype, A5 reads m
    # and writes hhat in fp32, A2/A6 read their inputs and write fp32 q, k and out)
    C, nc, sb = cfg.channels, cfg.n_comp, (2 if cfg.storage == "bf16" else 4)
    node_bytes = N * (2 * nc * C * sb + 8 * nc * C + 4 * nc * C + 8 * C)

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
                        f"{cfg.storage} storage (h' and m in fp16 under a per-node scale, q and k fp32), "
                        f"fp32 arithmetic",
            "nnz": nnz,
            "steps_per_s": 1e3 / ms_step,
            "timing": "HIP events on the main stream around the whole loop of --steps steps",
            "stage_ms": stage_ms,
            "arrangement": "projections + source coupling on a second stream during the neighbour build (which "
                           "also emits the Hilbert target order); attention + target coupling + output projection "
                           "after both",
            "one_stream_ms_per_step": one_stream_ms,
            "one_stream": "the same calls in stage order on one stream (stage_ms are taken on this arrangement)",
            "layer_ms_excl_neighbours": layer_ms,
            "layer_pairs_per_s_excl_neighbours": nnz / (layer_ms * 1e-3),
            "layer_steps_per_s_excl_neighbours": 1e3 / layer_ms,
            "layer_algorithmic_frac_excl_neighbours": (a["bytes"] + node_bytes) / (layer_ms * 1e-3)
                                                      / (HBM_PEAK_GBS * 1e9),
        },
        "roofline": roofline(cfg, nnz, t_attn_ms),
        "cpu_baseline": None,
    }
    if not args.no_per_config:
        rec["config"]["per_config"] = {}
        for name in PER_CONFIG:
            if name != cfg.name:
                rec["config"]["per_config"][name] = per_config(B, W, torch, name)
                torch.cuda.empty_cache()
    if not args.no_stack:
        rec["config"]["stack"] = stack_bench(B, W, torch)
    if not args.no_backward:
        rec["config"]["backward"] = backward_bench(B, W, torch)
    if not args.no_edge:
        rec["config"]["edge_form"] = edge_bench(B, W, torch)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
