"""Build libs6.so (the HIP library) for gfx950 with hipcc, in-tree.

    python -m selective_state_space_63_amd.build

Each source in csrc/ is compiled to an object in parallel (one hipcc per
file), then the objects are linked into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("scan.hip", "scan_ext.hip", "scan_conv.hip", "scan_hold.hip",
                                                    "step.hip", "bwd.hip", "ssd.hip", "common.hip")]
HEADERS = [os.path.join(CSRC, "s6_internal.h"), os.path.join(CSRC, "scan_kernel.h"),
           os.path.join(ROOT, "include", "s6.h")]
LIB = os.path.join(PKG, "libs6.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are switched off: hipcc would otherwise pair
# independent fp32 operations into v_pk_* forms.
# MFMA results go to VGPRs (the matrix-core kernels read them with VALU
# instructions; the accumulation-register form would add a copy per result).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include")]


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    tmpdir = tempfile.mkdtemp(prefix="s6build_")
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append((src, subprocess.Popen([HIPCC, *FLAGS, *(extra or []), "-c", "-o", obj, src],
                                            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = False
    for src, p in procs:
        o, e = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(f"--- {os.path.basename(src)}\n{o}{e}")
            failed = True
        elif verbose:
            sys.stderr.write(e)
    if failed:
        raise RuntimeError("hipcc failed building libs6.so")
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libs6.so failed")
    os.replace(tmp, out)
    for obj in objs:
        os.remove(obj)
    os.rmdir(tmpdir)
    return out


def asm(out: str, src: str = SOURCES[0], extra: list[str] | None = None) -> str:
    """Device assembly of one source file (for inspection)."""
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], *(extra or []),
           "--cuda-device-only", "-S", "-o", out, src]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
