"""MI355X (gfx950) KDA: chunked prefill and recurrent decode in HIP.

``chunk_fwd`` and ``recurrent_step`` call the C ABI of ``libkda.so``
(include/kda.h) through ctypes.  The library is loaded on first use and is
required: there is no CPU or PyTorch fallback.
"""
from .kda import (  # noqa: F401
    KDAError,
    Plan,
    chunk_bwd,
    chunk_bwd_workspace_size,
    chunk_fwd,
    chunk_fwd_noalloc,
    chunk_fwd_varlen,
    chunk_fwd_varlen_workspace_size,
    snapshot_count,
    chunk_plan,
    chunk_workspace_size,
    load_library,
    profile_start,
    profile_stop,
    recurrent_step,
    recurrent_steps,
    status_string,
    version,
)
from .build import LIB_PATH, build_library  # noqa: F401

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_bwd", "chunk_bwd_workspace_size", "chunk_fwd_varlen", "chunk_fwd_varlen_workspace_size", "snapshot_count", "recurrent_step", "recurrent_steps", "chunk_plan", "chunk_workspace_size", "profile_start", "profile_stop",
           "load_library", "build_library", "version", "status_string", "KDAError", "Plan"]
