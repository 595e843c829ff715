"""Build libs6.so (the HIP library) for gfx950 with hipcc, in-tree.

    python -m selective_state_space_63_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "s6.hip")
LIB = os.path.join(PKG, "libs6.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are switched off: hipcc would otherwise pair
# independent fp32 operations into v_pk_* forms.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libs6.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


def asm(out: str, extra: list[str] | None = None) -> str:
    """Device assembly of the library (for inspection)."""
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-fPIC", "-shared")], *(extra or []),
           "--cuda-device-only", "-S", "-o", out, SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
