"""Compile the HIP library (libinkattn.so) for gfx950, in-tree.

Run ``python -m transformer_attention_03_amd.build``.  hipcc cross-compiles
without a GPU.  Every HIP translation unit is built with packed-fp32 code
generation disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", "inkattn.hip"), os.path.join(PKG, "csrc", "attn_bwd.hip")]
LIB = os.path.join(PKG, "libinkattn.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag: drop that notice
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
