"""Compile the HIP library libkda.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
# KDA_LIBRARY: load another build of the library instead (the host sanitizer
# test's); build_library() always writes the in-tree libkda.so
BUILD_PATH = os.path.join(PKG, "libkda.so")
LIB_PATH = os.environ.get("KDA_LIBRARY") or BUILD_PATH
SOURCES = ["kda_api.cpp", "kda_chunk.hip", "kda_split.hip", "kda_decode.hip", "kda_bwd.hip", "kda_bwd_chunk.hip",
           "kda_noalloc.hip", "kda_fused.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda.so)")


def _compile(out: str, opt: list, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH] + opt + ["-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out_txt = (res.stdout + res.stderr).strip()
    # the host pass does not know the device-only feature flag
    lines = [ln for ln in out_txt.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    """Compile every source into libkda.so next to this file; returns its path."""
    return _compile(BUILD_PATH, ["-O3"], verbose)


def build_library_sanitized(path: str, verbose: bool = False) -> str:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code only (argument checks, plans, launch set-up; every report
    fatal), the device code as in build_library.  Loads only into a process
    that starts with clang's ASan runtime preloaded (asan_runtime())."""
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", f]
    return _compile(path, ["-O1", "-g", "-fno-omit-frame-pointer"] + san, verbose)


def asan_runtime() -> str:
    """clang's AddressSanitizer runtime that build_library_sanitized needs."""
    import glob
    root = os.path.dirname(os.path.dirname(hipcc()))
    cands = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not cands:
        raise RuntimeError("clang ASan runtime not found under " + root)
    return cands[-1]
