"""Builds libe2v2.so (HIP, gfx950) in the package directory.

    python -m atomistic_attention_amd.build

Every source is compiled with hipcc for gfx950 only.  Packed fp32 instructions
are disabled (-packed-fp32-ops) for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libe2v2.so")
SOURCES = ["e2v2_api.cpp", "eaas.hip", "proj.hip", "qkv_eaas.hip", "eaas_outproj.hip", "attn.hip", "attn_pair.hip", "attn_quad.hip",
           "neighbors.hip", "order.hip", "attn_bwd.hip", "attn_f32.hip", "edge.hip"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags(arch: str = "gfx950"):
    return ["-x", "hip", f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
            "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, arch: str = "gfx950", jobs: int = 5) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc, *flags(arch), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            procs[[p.poll() is None for _, p in procs].index(True)][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if out.strip() and (verbose or p.returncode):
            print(f"--- {src}\n{out}", file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={arch}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
