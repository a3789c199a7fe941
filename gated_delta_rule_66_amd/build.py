"""Compile the HIP library libkda.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_chunk.hip", "kda_split.hip", "kda_decode.hip", "kda_bwd.hip", "kda_bwd_chunk.hip",
           "kda_noalloc.hip", "kda_fused.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda.so)")


def build_library(verbose: bool = False) -> str:
    """Compile every source into libkda.so next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the device-only feature flag
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH
