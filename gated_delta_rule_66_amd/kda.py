"""ctypes binding of libkda.so (declared in include/kda.h).

Argument marshalling only: every step of KDA runs in the HIP kernels.  torch
supplies device memory (outputs, workspace) and the current HIP stream.  If
the library is not built this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from .build import LIB_PATH

KDA_OK = 0
KDA_ERR_INVALID_ARG = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE = 3
KDA_ERR_HIP = 4
KDA_F32 = 0
KDA_BF16 = 1

EXPORTED_SYMBOLS = (
    "kda_chunk_fwd_plan",
    "kda_chunk_fwd_workspace_size",
    "kda_chunk_fwd",
    "kda_chunk_fwd_planned_workspace_size",
    "kda_chunk_fwd_planned",
    "kda_chunk_fwd_noalloc",
    "kda_chunk_fwd_gated",
    "kda_chunk_fwd_varlen_workspace_size",
    "kda_chunk_fwd_varlen",
    "kda_chunk_fwd_varlen_gated",
    "kda_chunk_fwd_varlen_snapshots",
    "kda_recurrent_step",
    "kda_recurrent_steps",
    "kda_chunk_bwd_workspace_size",
    "kda_chunk_bwd",
    "kda_status_string",
    "kda_version",
    "kda_profile_start",
    "kda_profile_stop",
)


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


class Plan(ctypes.Structure):
    _fields_ = [("n_seg", ctypes.c_int), ("v_block", ctypes.c_int), ("split", ctypes.c_int)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libkda.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    i, p, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.kda_chunk_fwd_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.kda_chunk_fwd_plan.restype = i
    lib.kda_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd.restype = i
    lib.kda_chunk_fwd_planned_workspace_size.argtypes = [i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.kda_chunk_fwd_planned_workspace_size.restype = sz
    lib.kda_chunk_fwd_planned.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p,
                                          ctypes.POINTER(Plan), p, sz, p]
    lib.kda_chunk_fwd_planned.restype = i
    lib.kda_chunk_fwd_noalloc.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p, ctypes.POINTER(Plan), p]
    lib.kda_chunk_fwd_noalloc.restype = i
    lib.kda_chunk_fwd_gated.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p, p,
                                        ctypes.POINTER(Plan), p, sz, p]
    lib.kda_chunk_fwd_gated.restype = i
    lib.kda_chunk_fwd_varlen_gated.argtypes = [i, p, i, i, i, i, i, p, p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd_varlen_gated.restype = i
    lib.kda_chunk_fwd_varlen_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_chunk_fwd_varlen_workspace_size.restype = sz
    lib.kda_chunk_fwd_varlen.argtypes = [i, p, i, i, i, i, i, p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_fwd_varlen.restype = i
    lib.kda_chunk_fwd_varlen_snapshots.argtypes = [i, p, i, i, i, i, i, p, p, p, p, p, p, p, p, i, p, i, p, sz, p]
    lib.kda_chunk_fwd_varlen_snapshots.restype = i
    lib.kda_recurrent_step.argtypes = [i, i, i, i, i, p, p, p, p, p, p, p, p]
    lib.kda_recurrent_step.restype = i
    lib.kda_recurrent_steps.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p, p]
    lib.kda_recurrent_steps.restype = i
    lib.kda_chunk_bwd_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.kda_chunk_bwd_workspace_size.restype = sz
    lib.kda_chunk_bwd.argtypes = [i, i, i, i, i, i] + [p] * 14 + [p, sz, p]
    lib.kda_chunk_bwd.restype = i
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_char_p
    lib.kda_profile_start.argtypes = [i]
    lib.kda_profile_start.restype = i
    lib.kda_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), i]
    lib.kda_profile_stop.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def version() -> str:
    return load_library().kda_version().decode()


def profile_start(max_launches: int = 4096) -> None:
    """Start per-launch event timing of the library's kernels (``kda_profile_start``)."""
    st = load_library().kda_profile_start(int(max_launches))
    if st != KDA_OK:
        raise KDAError(st, "kda_profile_start")


def profile_stop(cap: int = 4096):
    """Stop timing; returns [(launch name, milliseconds)] in launch order."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = load_library().kda_profile_stop(names, ms, int(cap))
    if n < 0:
        raise RuntimeError("kda_profile_stop failed (profiling not started or event query failed)")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError("KDA inputs must be bfloat16 or float32, got %s" % dt)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _plan_arg(plan) -> Optional[Plan]:
    """None, a Plan, or a tuple (n_seg, v_block[, split]); 0 = library's choice."""
    if plan is None:
        return None
    if isinstance(plan, Plan):
        return plan
    vals = [int(x) for x in plan]
    if len(vals) not in (2, 3):
        raise ValueError("plan is (n_seg, v_block[, split])")
    return Plan(vals[0], vals[1], vals[2] if len(vals) == 3 else 0)


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def chunk_plan(B: int, T: int, H: int, K: int, V: int, dtype: torch.dtype) -> Tuple[int, int, int]:
    """(n_seg, v_block, split) the library picks for these sizes on the current device."""
    pl = Plan()
    st = load_library().kda_chunk_fwd_plan(B, T, H, K, V, _dtype_code(dtype), ctypes.byref(pl))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_plan")
    return pl.n_seg, pl.v_block, pl.split


def chunk_workspace_size(B: int, T: int, H: int, K: int, V: int, dtype: torch.dtype, plan=None) -> int:
    """Workspace bytes of ``kda_chunk_fwd`` (plan None: the library's plan) or
    of ``kda_chunk_fwd_planned`` in ``plan``."""
    pl = _plan_arg(plan)
    lib = load_library()
    if pl is None:
        n = lib.kda_chunk_fwd_workspace_size(B, T, H, K, V, _dtype_code(dtype))
    else:
        n = lib.kda_chunk_fwd_planned_workspace_size(B, T, H, K, V, _dtype_code(dtype), ctypes.byref(pl))
    if n == ctypes.c_size_t(-1).value:
        raise KDAError(KDA_ERR_INVALID_ARG, "kda_chunk_fwd_workspace_size")
    return int(n)


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              output_final_state: bool = True, plan=None, *,
              out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None):
    """KDA chunked prefill through ``kda_chunk_fwd`` (``kda_chunk_fwd_planned``
    with a ``plan``, ``kda_chunk_fwd_gated`` with ``gate``).

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H] (one dtype, bf16
    or fp32, on one GPU); initial_state: [B, H, K, V] fp32 or None.
    Returns (o [B, T, H, V], final_state [B, H, K, V] fp32 or None).
    ``final_state`` may be passed to write in place (it may be
    ``initial_state`` itself); ``plan`` = (n_seg, v_block, split), 0 = auto.
    ``gate``: [B, T, H, V] output gate pre-activation; o is returned as
    o * sigmoid(gate).
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("beta", beta, (B, T, H))):
        _check(t, name, shp, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, K, V), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, V), dtype=dt, device=dev)
    else:
        _check(out, "out", (B, T, H, V), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", (B, H, K, V), torch.float32, dev)
    pl = _plan_arg(plan)
    ws_bytes = chunk_workspace_size(B, T, H, K, V, dt, pl)
    if ws_bytes > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gate is not None:
        _check(gate, "gate", (B, T, H, V), dt, dev)
        st = load_library().kda_chunk_fwd_gated(
            B, T, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate),
            _ptr(initial_state), _ptr(out), _ptr(final_state),
            None if pl is None else ctypes.byref(pl), _ptr(workspace), ws_len, _stream_ptr(dev))
        if st != KDA_OK:
            raise KDAError(st, "kda_chunk_fwd_gated")
        return out, final_state
    if pl is None:
        st = load_library().kda_chunk_fwd(
            B, T, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace), ws_len, _stream_ptr(dev))
        if st != KDA_OK:
            raise KDAError(st, "kda_chunk_fwd")
        return out, final_state
    st = load_library().kda_chunk_fwd_planned(
        B, T, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(initial_state), _ptr(out), _ptr(final_state), ctypes.byref(pl), _ptr(workspace), ws_len,
        _stream_ptr(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_planned")
    return out, final_state


NOALLOC_SCRATCH_BYTES = 64 << 20


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, initial_state: Optional[torch.Tensor], *, out: torch.Tensor,
                      final_state: Optional[torch.Tensor] = None, plan=None):
    """Prefill through ``kda_chunk_fwd_noalloc``: no workspace argument and no
    allocation here or in the library (the caller passes ``out`` and, if
    wanted, ``final_state``; it may be ``initial_state``).  ``plan`` as in
    ``chunk_fwd``.  Returns (out, final_state)."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("beta", beta, (B, T, H)), ("out", out, (B, T, H, V))):
        _check(t, name, shp, dt, dev)
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _check(t, name, (B, H, K, V), torch.float32, dev)
    pl = _plan_arg(plan)
    st = load_library().kda_chunk_fwd_noalloc(
        B, T, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
        _ptr(out), _ptr(final_state), None if pl is None else ctypes.byref(pl), _stream_ptr(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_noalloc")
    return out, final_state


def chunk_fwd_varlen_workspace_size(N: int, T_total: int, H: int, K: int, V: int, dtype: torch.dtype) -> int:
    n = load_library().kda_chunk_fwd_varlen_workspace_size(N, T_total, H, K, V, _dtype_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise KDAError(KDA_ERR_INVALID_ARG, "kda_chunk_fwd_varlen_workspace_size")
    return int(n)


def snapshot_count(cu_seqlens, snapshot_interval: int) -> int:
    """Snapshots a packed batch yields: sum_i floor(len_i / snapshot_interval)
    (cu_seqlens as a host sequence or tensor; a device tensor is copied)."""
    cu = [int(x) for x in (cu_seqlens.tolist() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens)]
    return sum(max(0, b - a) // snapshot_interval for a, b in zip(cu[:-1], cu[1:]))


def chunk_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, cu_seqlens: torch.Tensor,
                     initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True, *,
                     out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, snapshot_interval: int = 0,
                     snapshots: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None):
    """Packed variable-length prefill through ``kda_chunk_fwd_varlen`` (or
    ``kda_chunk_fwd_varlen_snapshots`` when ``snapshot_interval`` > 0).

    q, k, g: [T_total, H, K]; v: [T_total, H, V]; beta: [T_total, H] (bf16 or
    fp32); cu_seqlens: int32 [N + 1] on the same device; initial_state:
    [N, H, K, V] fp32 or None.  Returns (o [T_total, H, V], final_state
    [N, H, K, V] or None); ``final_state`` may be ``initial_state`` itself.
    With ``snapshot_interval`` (a multiple of 64) it returns (o, final_state,
    snapshots [S, H, K, V] fp32): snapshot m of sequence i, the state after
    its first (m + 1) * snapshot_interval tokens, sits at
    snapshot_count(cu_seqlens[:i + 1], snapshot_interval) + m.  ``snapshots``
    may be passed preallocated (its first dimension is the capacity).
    ``gate``: [T_total, H, V] output gate pre-activation (o * sigmoid(gate));
    not together with snapshots.
    """
    T_total, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (T_total, H, K)), ("k", k, (T_total, H, K)), ("g", g, (T_total, H, K)),
                         ("v", v, (T_total, H, V)), ("beta", beta, (T_total, H))):
        _check(t, name, shp, dt, dev)
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, K, V), torch.float32, dev)
    if out is None:
        out = torch.empty((T_total, H, V), dtype=dt, device=dev)
    else:
        _check(out, "out", (T_total, H, V), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", (N, H, K, V), torch.float32, dev)
    ws_bytes = chunk_fwd_varlen_workspace_size(N, T_total, H, K, V, dt)
    if ws_bytes > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gate is not None:
        if snapshot_interval:
            raise ValueError("gate and snapshots are separate calls")
        _check(gate, "gate", (T_total, H, V), dt, dev)
        st = load_library().kda_chunk_fwd_varlen_gated(
            N, _ptr(cu_seqlens), T_total, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
            _ptr(beta), _ptr(gate), _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace), ws_len,
            _stream_ptr(dev))
        if st != KDA_OK:
            raise KDAError(st, "kda_chunk_fwd_varlen_gated")
        return out, final_state
    if snapshot_interval:
        if snapshots is None:
            snapshots = torch.empty((snapshot_count(cu_seqlens, snapshot_interval), H, K, V),
                                    dtype=torch.float32, device=dev)
        else:
            _check(snapshots, "snapshots", (snapshots.shape[0], H, K, V), torch.float32, dev)
        st = load_library().kda_chunk_fwd_varlen_snapshots(
            N, _ptr(cu_seqlens), T_total, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
            _ptr(beta), _ptr(initial_state), _ptr(out), _ptr(final_state), int(snapshot_interval),
            _ptr(snapshots), snapshots.shape[0], _ptr(workspace), ws_len, _stream_ptr(dev))
        if st != KDA_OK:
            raise KDAError(st, "kda_chunk_fwd_varlen_snapshots")
        return out, final_state, snapshots
    st = load_library().kda_chunk_fwd_varlen(
        N, _ptr(cu_seqlens), T_total, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(workspace), ws_len, _stream_ptr(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_varlen")
    return out, final_state


def chunk_bwd_workspace_size(B: int, T: int, H: int, K: int, V: int, dtype: torch.dtype) -> int:
    n = load_library().kda_chunk_bwd_workspace_size(B, T, H, K, V, _dtype_code(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise KDAError(KDA_ERR_INVALID_ARG, "kda_chunk_bwd_workspace_size")
    return int(n)


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              initial_state: Optional[torch.Tensor], d_o: Optional[torch.Tensor],
              d_final_state: Optional[torch.Tensor] = None, *, want_d_initial_state: bool = True,
              workspace: Optional[torch.Tensor] = None):
    """Gradients of the prefill through ``kda_chunk_bwd``.

    Inputs as ``chunk_fwd``; d_o: [B, T, H, V] (dL/do) or None; d_final_state:
    [B, H, K, V] fp32 (dL/dS_T) or None.  Returns (dq, dk, dv, dg, dbeta,
    d_initial_state or None), gradients in the input dtype, the last fp32.
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("beta", beta, (B, T, H))):
        _check(t, name, shp, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, K, V), torch.float32, dev)
    if d_o is not None:
        _check(d_o, "d_o", (B, T, H, V), dt, dev)
    if d_final_state is not None:
        _check(d_final_state, "d_final_state", (B, H, K, V), torch.float32, dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    ds0 = torch.empty((B, H, K, V), dtype=torch.float32, device=dev) if want_d_initial_state else None
    ws_bytes = chunk_bwd_workspace_size(B, T, H, K, V, dt)
    if ws_bytes > 0 and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().kda_chunk_bwd(
        B, T, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
        _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(ds0),
        _ptr(workspace), ws_len, _stream_ptr(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_bwd")
    return dq, dk, dv, dg, dbeta, ds0


def recurrent_steps(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, state: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                    step_states=None):
    """T tokens per sequence through ``kda_recurrent_steps`` (multi-token
    verification); ``state`` is updated in place to the state after the last
    token.  q, k, g: [N, T, H, K]; v: [N, T, H, V]; beta: [N, T, H]; state:
    [N, H, K, V] fp32.  ``step_states``: None, True (allocate) or a
    [N, T, H, K, V] fp32 tensor that receives the state after every token.
    Returns o [N, T, H, V], or (o, step_states) when step states are asked for."""
    N, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (N, T, H, K)), ("k", k, (N, T, H, K)), ("g", g, (N, T, H, K)),
                         ("v", v, (N, T, H, V)), ("beta", beta, (N, T, H))):
        _check(t, name, shp, dt, dev)
    _check(state, "state", (N, H, K, V), torch.float32, dev)
    if out is None:
        out = torch.empty((N, T, H, V), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, T, H, V), dt, dev)
    want_steps = step_states is not None and step_states is not False
    if step_states is True:
        step_states = torch.empty((N, T, H, K, V), dtype=torch.float32, device=dev)
    elif want_steps:
        _check(step_states, "step_states", (N, T, H, K, V), torch.float32, dev)
    st = load_library().kda_recurrent_steps(N, T, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                            _ptr(beta), _ptr(state), _ptr(out),
                                            _ptr(step_states) if want_steps else None, _stream_ptr(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_recurrent_steps")
    return (out, step_states) if want_steps else out


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   beta: torch.Tensor, state: torch.Tensor, *, out: Optional[torch.Tensor] = None):
    """One KDA decode step through ``kda_recurrent_step``; ``state`` is
    updated in place.  q, k, g: [N, H, K]; v: [N, H, V]; beta: [N, H];
    state: [N, H, K, V] fp32.  Returns o [N, H, V]."""
    N, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (N, H, K)), ("k", k, (N, H, K)), ("g", g, (N, H, K)),
                         ("v", v, (N, H, V)), ("beta", beta, (N, H))):
        _check(t, name, shp, dt, dev)
    _check(state, "state", (N, H, K, V), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, V), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, H, V), dt, dev)
    st = load_library().kda_recurrent_step(N, H, K, V, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(g), _ptr(beta), _ptr(state), _ptr(out),
                                           _stream_ptr(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_recurrent_step")
    return out
