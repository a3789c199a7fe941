"""ctypes marshalling for the fp64 KDA oracle (``kda_oracle.c``).

Test infrastructure: see the package docstring.  Inputs may be numpy arrays
or CPU torch tensors of any float dtype whose values are exactly representable
in fp32 (bf16 and fp32 inputs are); they are passed as fp32 and every
operation inside the oracle is fp64.  The initial state is passed as fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(_HERE, "kda_oracle.c")
# KDA_ORACLE_LIBRARY: another build of kda_oracle.c to load instead (the
# sanitizer test's ASan/UBSan build); it is not rebuilt here
ORACLE_SO = os.environ.get("KDA_ORACLE_LIBRARY") or os.path.join(_HERE, "libkda_oracle.so")

_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, fp64, OpenMP, no fast-math)."""
    if not force and os.path.exists(ORACLE_SO):
        return ORACLE_SO
    tmp = ORACLE_SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", tmp, ORACLE_SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, ORACLE_SO)
    return ORACLE_SO


def build_oracle_sanitized(path: str) -> str:
    """Compile the oracle with gcc's AddressSanitizer and UndefinedBehavior-
    Sanitizer (every report fatal) into `path`, for the host sanitizer test."""
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", path, ORACLE_SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(ORACLE_SO):
            build_oracle(force=True)
        lib = ctypes.CDLL(ORACLE_SO)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [i, i, i, i, i, p, p, p, p, p, p, p, p, i]
        lib.kda_oracle_fwd.restype = i
        lib.kda_oracle_step.argtypes = [i, i, i, i, p, p, p, p, p, p, p, i]
        lib.kda_oracle_step.restype = i
        lib.kda_oracle_bwd.argtypes = [i, i, i, i, i, p, p, p, p, p, p, p, p, p, p, p, p, p, p, i]
        lib.kda_oracle_bwd.restype = i
        lib.kda_oracle_max_threads.argtypes = []
        lib.kda_oracle_max_threads.restype = i
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu().float().numpy()
    a = np.ascontiguousarray(np.asarray(x), dtype=np.float32)
    return a


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def oracle_max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def oracle_fwd(q, k, v, g, beta, s0=None, *, want_o=True, want_state=True,
               nthreads: int = 0):
    """Token-by-token fp64 KDA forward.

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H];
    s0: [B, H, K, V] or None (zeros).
    Returns (o [B,T,H,V] fp64 or None, sT [B,H,K,V] fp64 or None).
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    s0 = _f64(s0)
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and g.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V) and beta.shape == (B, T, H)
    if s0 is not None:
        assert s0.shape == (B, H, K, V)
    o = np.zeros((B, T, H, V), np.float64) if want_o else None
    sT = np.zeros((B, H, K, V), np.float64) if want_state else None
    rc = _load().kda_oracle_fwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(g), _ptr(beta), _ptr(s0), _ptr(o),
                                _ptr(sT), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected sizes")
    return o, sT


def oracle_step(q, k, v, g, beta, state, *, nthreads: int = 0):
    """One decode step, state [N,H,K,V] fp64 updated IN PLACE.

    q, k, g: [N, H, K]; v: [N, H, V]; beta: [N, H].  Returns o [N, H, V].
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    N, H, K = q.shape
    V = v.shape[-1]
    assert isinstance(state, np.ndarray) and state.dtype == np.float64
    assert state.shape == (N, H, K, V) and state.flags.c_contiguous
    o = np.zeros((N, H, V), np.float64)
    rc = _load().kda_oracle_step(N, H, K, V, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                                 int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected sizes")
    return o


def oracle_bwd(q, k, v, g, beta, s0, d_o, dsT=None, *, nthreads: int = 0):
    """Token-by-token fp64 KDA backward (reverse-mode chain rule of
    ``oracle_fwd``).

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H]; s0: [B, H, K, V]
    or None; d_o: [B, T, H, V] (dL/do) or None (zeros); dsT: [B, H, K, V]
    (dL/dS_T) or None (zeros).
    Returns (dq, dk, dv, dg, dbeta, ds0), fp64 in the input layouts.
    """
    q, k, v, g, beta, d_o = (_f32(x) for x in (q, k, v, g, beta, d_o))
    s0, dsT = _f64(s0), _f64(dsT)
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, T, H, K) and g.shape == (B, T, H, K)
    assert v.shape == (B, T, H, V) and beta.shape == (B, T, H)
    for name, t, shp in (("s0", s0, (B, H, K, V)), ("d_o", d_o, (B, T, H, V)), ("dsT", dsT, (B, H, K, V))):
        if t is not None:
            assert t.shape == shp, name
    dq = np.zeros((B, T, H, K), np.float64)
    dk = np.zeros((B, T, H, K), np.float64)
    dv = np.zeros((B, T, H, V), np.float64)
    dg = np.zeros((B, T, H, K), np.float64)
    dbeta = np.zeros((B, T, H), np.float64)
    ds0 = np.zeros((B, H, K, V), np.float64)
    rc = _load().kda_oracle_bwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                _ptr(d_o), _ptr(dsT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                                _ptr(ds0), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected sizes (%d)" % rc)
    return dq, dk, dv, dg, dbeta, ds0
