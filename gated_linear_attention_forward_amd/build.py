"""Builds libgla.so (the C-ABI library of include/gla.h) in-tree for gfx950.

Usage: python -m gated_linear_attention_forward_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgla.so")
ARCH = "gfx950"

# Packed fp32 arithmetic stays off: the compiler must not form v_pk_*_f32.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC"]
# The forward kernels read their MFMA results with ordinary vector ALU
# instructions (the epilogue, the partial-state stores): keeping those results
# in VGPRs instead of AGPRs saves a v_accvgpr_read per result.
FILE_FLAGS = {"gla_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in ("gla_kernels.hip", "gla_softmax.hip", "gla_backward.hip", "gla_project.hip",
                "gla_probe.hip"):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run(["hipcc", *HIP_FLAGS, *FILE_FLAGS.get(src, []), f"-I{INCLUDE}", f"-I{CSRC}", "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    aobj = os.path.join(BUILD, "gla_api.o")
    _run(["hipcc", *HOST_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
          os.path.join(CSRC, "gla_api.cpp"), "-o", aobj], verbose)
    tmp = LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, aobj, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
