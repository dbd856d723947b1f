"""Build liboscar.so (HIP, gfx950) in-tree with hipcc.

Run ``python -m bit_rotated_kv_attn_amd.build``.  The library is written next
to this file, and the Python binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["csrc/abi.hip", "csrc/quantize.hip", "csrc/decode.hip"]
LIB = os.path.join(PKG, "liboscar.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liboscar)")


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", f"-I{os.path.join(ROOT, 'include')}",
            # packed FP32 instructions stay disabled for every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-o", out] + [os.path.join(PKG, s) for s in SOURCES]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"       # hipcc's host pass does not know the device feature
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
