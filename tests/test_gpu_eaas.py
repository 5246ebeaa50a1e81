"""e2v2_eaas_couple (the EAAS kernel) against the oracle's dense Clebsch-Gordan
tensor product (E2Former-V2 explainer, section 2.3, Proposition 4.3)."""
import numpy as np
import pytest
import torch

from atomistic_attention_amd import workloads as W
from oracle import so3
from tests._helpers import bf16_close, f32, record, rel_err, to_storage

pytestmark = pytest.mark.gpu


def _inputs(n, L, C, seed):
    rng = np.random.default_rng(seed)
    pos = rng.uniform(-30, 30, (n, 3))
    pos[0] = 0.0                       # no direction
    pos[1] = [0, 0, 7.5]               # +z: alpha undefined, beta = 0
    pos[2] = [0, 0, -2.25]             # -z: beta = pi
    pos[3] = [1e-3, 0, 0]
    pos = pos.astype(np.float32).astype(np.float64)
    x = rng.standard_normal((n, (L + 1) ** 2, C))
    w = rng.standard_normal((len(so3.paths(L)), C)).astype(np.float32).astype(np.float64)
    return pos, x, w


@pytest.mark.parametrize("L", [0, 1, 2, 3])
@pytest.mark.parametrize("C", [32, 128])
def test_eaas_fp32_matches_full_cg(gpu_lib, L, C):
    n = 301                            # several blocks and a ragged tail
    pos, x, w = _inputs(n, L, C, 10 * L + C)
    x = x.astype(np.float32).astype(np.float64)
    y = gpu_lib.e2v2_eaas_couple(f32(pos), f32(x), f32(w), L).cpu().numpy()
    ref = so3.tensor_product(x, pos, w, L)
    record(f"eaas_fp32[{L},{C}]", err=rel_err(y, ref))
    assert rel_err(y, ref) < 1e-5


@pytest.mark.parametrize("L", [2, 3])
def test_eaas_bf16_io(gpu_lib, L):
    n, C = 257, 128
    pos, x, w = _inputs(n, L, C, 99 + L)
    xb = W.round_bf16(x)
    ref = so3.tensor_product(xb, pos, w, L)
    y = gpu_lib.e2v2_eaas_couple(f32(pos), to_storage(xb, torch.bfloat16), f32(w), L).cpu().numpy()
    assert rel_err(y, ref) < 1e-5
    yb = gpu_lib.e2v2_eaas_couple(f32(pos), to_storage(xb, torch.bfloat16), f32(w), L,
                                  out_dtype=torch.bfloat16).float().cpu().numpy()
    record(f"eaas_bf16[{L}]", fp32_out=rel_err(y, ref), bf16_out=rel_err(yb, ref))
    assert bf16_close(yb, ref)                      # one bf16 rounding of the output
