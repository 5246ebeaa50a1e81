"""Shared helpers for the GPU tests: upload a seeded workload, error metric."""
from __future__ import annotations

import numpy as np
import torch

from atomistic_attention_amd import workloads as W


def storage_dtype(wl) -> torch.dtype:
    return torch.bfloat16 if wl.cfg.storage == "bf16" else torch.float32


def to_storage(a: np.ndarray, dt: torch.dtype, dev="cuda") -> torch.Tensor:
    if dt == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(W.bf16_bits(a)).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def f32(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def upload(wl, dev="cuda"):
    return W.device_arrays(wl, dev)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def bf16_close(got, ref, rms_floor=1e-5) -> bool:
    """Element-wise bound for one round-to-nearest bf16 store of an fp32 result:
    |got - ref| <= 2^-8 |ref| (half an ulp of an 8-bit significand) plus a small
    absolute floor for the fp32 arithmetic before the store."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return bool(np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + rms_floor * rms))


def fp16_close(got, ref, rms_floor=1e-5) -> bool:
    """Element-wise bound for one round-to-nearest fp16 store (under a power-of-two
    scale, which is exact) of an fp32 result: |got - ref| <= 2^-11 |ref| (half an
    ulp of an 11-bit significand) plus a small absolute floor, relative to the RMS,
    for the fp32 arithmetic before the store and for values in fp16's subnormal
    range below the node's scale."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return bool(np.all(np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) + rms_floor * rms))


def record(test: str, **vals):
    """Append measured parity numbers to $E2V2_PARITY_LOG (JSON lines), if set."""
    import json
    import os
    path = os.environ.get("E2V2_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": test, **{k: float(v) for k, v in vals.items()}}) + "\n")


def rows_from_device(start, length, idx):
    s = start.cpu().numpy().astype(np.int64)
    ln = length.cpu().numpy().astype(np.int64)
    ix = idx.cpu().numpy()
    return [ix[s[i]:s[i] + ln[i]] for i in range(s.size)]


def csr_from_rows(rows, dev="cuda"):
    lens = np.array([r.size for r in rows], dtype=np.int32)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    idx = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(start), t(lens), t(idx)


def tolerance(wl) -> float:
    """Max-abs error relative to the oracle output RMS (fp32: 1e-4, bf16 storage: 2e-2)."""
    return 2e-2 if wl.cfg.storage == "bf16" else 1e-4
