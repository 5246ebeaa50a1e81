"""The allocation-free forward (e2v2_attn_forward_noalloc) through the C ABI
against e2v2_attn_forward with a caller workspace, on the same inputs: the
same kernels on the same data, so the outputs are bit-identical.  Two calls in
a row on the library's one device array, the second with a smaller input."""
import numpy as np
import pytest
import torch

from atomistic_attention_amd import workloads as W
from tests._helpers import upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("storage", ["bf16", "fp32"])
def test_noalloc_forward_matches_workspace_forward(gpu_lib, storage):
    outs = []
    for n in (3000, 1200):                      # the second call is smaller than the first
        base = W.make_workload("c3", n=n)
        wl = W.make_workload(W.LayerConfig(**{**base.cfg.__dict__, "storage": storage}))
        c = wl.cfg
        d = upload(wl)
        desc = gpu_lib.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, d["dtype"])
        order = torch.empty(c.n, dtype=torch.int32, device="cuda")
        s, ln, ix, _ = gpu_lib.e2v2_build_neighbors(d["pos"], c.cutoff, c.max_neighbors, order_out=order)
        print(f"noalloc {storage} n={n}", flush=True)
        ref = gpu_lib.e2v2_attn_forward(desc, d["pos"], d["h"], d["weights"], s, ln, ix, target_order=order)
        got = torch.full_like(ref, float("nan"))
        gpu_lib.e2v2_attn_forward_noalloc(desc, d["pos"], d["h"], d["weights"], s, ln, ix, got, target_order=order)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert torch.isfinite(got).all() and float(got.abs().max()) > 0
        outs.append(got)
    assert outs[0].shape[0] == 3000 and outs[1].shape[0] == 1200


def test_noalloc_forward_rejects_a_workspace_beyond_its_array(gpu_lib):
    wl = W.make_workload("c3", n=64)
    c = wl.cfg
    d = upload(wl)
    desc = gpu_lib.make_desc(c.lmax, c.channels, c.heads, c.n_rbf, c.cutoff, d["dtype"])
    big = 200000                                # needs > 64 MiB
    assert gpu_lib.attn_workspace_bytes(desc, big) > 64 << 20
    pos = torch.zeros((big, 3), dtype=torch.float32, device="cuda")
    h = torch.zeros((big, c.n_comp, c.channels), dtype=d["dtype"], device="cuda")
    z = torch.zeros(big, dtype=torch.int32, device="cuda")
    out = torch.zeros((big, c.n_comp, c.channels), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.E2V2Error) as ei:
        gpu_lib.e2v2_attn_forward_noalloc(desc, pos, h, d["weights"], z, z, z, out)
    assert ei.value.status == gpu_lib.E2V2_ERR_CAPACITY
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0        # nothing ran
