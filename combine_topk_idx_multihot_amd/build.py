"""Build libmoe_mi355x.so (HIP, gfx950 only) in-tree, and beside it
libmoe_ceiling.so, the reference kernels a benchmark times against it.

    python -m combine_topk_idx_multihot_amd.build

The library is one shared object compiled by hipcc from csrc/*.hip against
include/moe_mi355x.h; the reference kernels come from ceiling_src/ceiling.hip
against include/moe_ceiling.h.  Packed-fp32 instruction selection is turned off for the
device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host
pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libmoe_mi355x.so")
CEILING_SRC = os.path.join(PKG, "ceiling_src", "ceiling.hip")
CEILING_LIB = os.path.join(LIB_DIR, "libmoe_ceiling.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(out: str, srcs: list[str], verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {out}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    _hipcc(LIB, sources(), verbose)
    _hipcc(CEILING_LIB, [CEILING_SRC], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(CEILING_LIB)
