"""Compile libmla_sparse.so for gfx950 in-tree with hipcc.

Usage: python -m sparse_latent_attention_amd.build [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_sparse.so")
SOURCES = ["mla_sparse.cpp", "mla_bf16.hip", "mla_f32.hip", "mla_noalloc.hip", "mla_append.hip", "mla_project.hip", "mla_explicit.hip", "mla_dequant.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-fvisibility=hidden",
    # packed fp32 vector ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments preloaded into scalar registers: the leading scalar
    # parameters of each kernel (up to the 16 registers the hardware allows)
    # are there when a workgroup starts, so its first loads do not wait for a
    # kernel-argument load
    "-mllvm", "-amdgpu-kernarg-preload-count=11",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and (res.stdout or res.stderr):
        sys.stderr.write(res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
