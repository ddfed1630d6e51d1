"""Builds libmssm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m selective_state_space_52_amd.build
The library is written next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmssm.so")
OBJDIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
SOURCES = ["scan_fwd.hip", "scan_fwd_n1_8.hip", "scan_fwd_n16.hip",
           "scan_fwd_n32.hip", "scan_fwd_n64.hip", "scan_fwd_n128.hip",
           "scan_bwd.hip", "state_update.hip", "conv1d.hip", "mamba2.hip",
           "noalloc.hip", "probe.hip", "mssm_api.cpp"]

# Packed fp32 VALU forms are switched off for every device compilation.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=" + ARCH,
          "-I" + INCLUDE, "-I" + CSRC, "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(force: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libmssm.so."""
    if not force and os.path.exists(LIB):
        return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


def asm(src: str = "scan_fwd.hip", out: str = None) -> str:
    """gfx950 assembly of one source (for reading the library's own generated code)."""
    out = out or os.path.join(OBJDIR, os.path.basename(src) + ".s")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [hipcc(), "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out] \
        + COMMON + DEVICE_FLAGS
    subprocess.check_call(cmd)
    return out


if __name__ == "__main__":
    print(build(force=True))
    if len(sys.argv) > 1 and sys.argv[1] == "--asm":
        print(asm())
