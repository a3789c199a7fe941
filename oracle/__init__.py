"""fp64 CPU oracle for KDA (Kimi Delta Attention).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  It shares no code with
the HIP library in ``gated_delta_rule_66_amd`` and never imports it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, token by token);
this module only compiles it with gcc and marshals numpy arrays.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    oracle_fwd,
    oracle_bwd,
    oracle_step,
    oracle_max_threads,
    ORACLE_SO,
)
