"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, and rejects bad arguments on the host before any HIP
call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_66_amd as kda_pkg
from gated_delta_rule_66_amd import kda as K_

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1
FAKE = 1 << 20          # an aligned, never-dereferenced address


def _lib():
    if not os.path.exists(kda_pkg.LIB_PATH):
        kda_pkg.build_library()
    return K_.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kda_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_expected_calls():
    decl = _declared_functions()
    assert decl == sorted(K_.EXPORTED_SYMBOLS), decl


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = os.popen("nm -D --defined-only %s" % kda_pkg.LIB_PATH).read()
    for name in _declared_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_version_and_status_strings():
    _lib()
    assert "gfx950" in kda_pkg.version()
    for s in range(5):
        assert kda_pkg.status_string(s) and kda_pkg.status_string(s) != "unknown status"
    assert kda_pkg.status_string(99) == "unknown status"


def _fwd(lib, B=1, T=64, H=1, K=128, V=128, dt=BF16, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
         s0=None, o=FAKE, sT=None, plan=None, ws=None, ws_bytes=0):
    """kda_chunk_fwd (library plan), or kda_chunk_fwd_planned with `plan`."""
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    if plan is None:
        return lib.kda_chunk_fwd(B, T, H, K, V, dt, p(q), p(k), p(v), p(g), p(beta), p(s0), p(o), p(sT),
                                 p(ws), ws_bytes, None)
    return lib.kda_chunk_fwd_planned(B, T, H, K, V, dt, p(q), p(k), p(v), p(g), p(beta), p(s0), p(o), p(sT),
                                     ctypes.byref(plan), p(ws), ws_bytes, None)


def _ws(lib, B, T, H, K, V, dt, plan=None):
    if plan is None:
        return lib.kda_chunk_fwd_workspace_size(B, T, H, K, V, dt)
    return lib.kda_chunk_fwd_planned_workspace_size(B, T, H, K, V, dt, ctypes.byref(plan))


# The prototypes of the hot-path boundary, as fixed for this library: the two
# calls of the path (prefill with optional initial and final state, one decode
# step), the workspace query, status strings and version.
BOUNDARY_PROTOTYPES = {
    "kda_chunk_fwd_workspace_size":
        "size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt);",
    "kda_chunk_fwd":
        "kda_status kda_chunk_fwd(int B, int T, int H, int K, int V, kda_dtype dt, "
        "const void* q, const void* k, const void* v, const void* g, const void* beta, "
        "const float* initial_state, void* o, float* final_state, void* workspace, size_t workspace_bytes, "
        "hipStream_t stream);",
    "kda_recurrent_step":
        "kda_status kda_recurrent_step(int N, int H, int K, int V, kda_dtype dt, "
        "const void* q, const void* k, const void* v, const void* g, const void* beta, "
        "float* state, void* o, hipStream_t stream);",
    "kda_status_string": "const char* kda_status_string(kda_status s);",
    "kda_version": "const char* kda_version(void);",
}


def _declaration(src, name):
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    m = re.search(r"^[^;{}#]*?\b%s\s*\([^;]*\);" % name, src, flags=re.M)
    assert m, name
    return " ".join(m.group(0).split()).replace("( ", "(").replace(" )", ")")


def test_boundary_prototypes_verbatim():
    src = open(HEADER).read()
    for name, proto in BOUNDARY_PROTOTYPES.items():
        assert _declaration(src, name) == proto, (name, _declaration(src, name))
    # the status and dtype codes
    body = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    for code, val in (("KDA_OK", 0), ("KDA_ERR_INVALID_ARG", 1), ("KDA_ERR_UNSUPPORTED", 2),
                      ("KDA_ERR_WORKSPACE", 3), ("KDA_ERR_HIP", 4), ("KDA_F32", 0), ("KDA_BF16", 1)):
        assert re.search(r"\b%s\s*=\s*%d\b" % (code, val), body), code


def test_prefill_rejects_bad_sizes_before_any_launch():
    lib = _lib()
    assert _fwd(lib, B=-1) == INVALID
    assert _fwd(lib, T=-5) == INVALID
    assert _fwd(lib, H=-1) == INVALID
    assert _fwd(lib, K=0) == INVALID
    assert _fwd(lib, dt=7) == INVALID
    assert _fwd(lib, K=96) == UNSUPPORTED
    assert _fwd(lib, V=256) == UNSUPPORTED


def test_fp32_at_128_takes_the_token_serial_form():
    # no chunk kernels for fp32 with K = 128: the plan is the token-serial
    # form (split 3, one segment, 64-column blocks), chosen without a device
    # query and with no workspace (fp32 at K = 64, V = 128 runs the
    # single-pass chunk kernel in 64-column blocks)
    lib = _lib()
    for K, V in ((128, 128), (128, 64)):
        pl = K_.Plan()
        assert lib.kda_chunk_fwd_plan(2, 1000, 3, K, V, F32, ctypes.byref(pl)) == OK
        assert (pl.n_seg, pl.v_block, pl.split) == (1, 64, 3)
        assert _ws(lib, 2, 1000, 3, K, V, F32) == 0
        assert lib.kda_chunk_fwd_varlen_workspace_size(4, 1000, 3, K, V, F32) == 0
    # the token-serial form has one segment and 64-column blocks only
    for bad in (K_.Plan(2, 64, 3), K_.Plan(1, 128, 3)):
        assert _fwd(lib, plan=bad) == UNSUPPORTED
        assert _ws(lib, 1, 64, 1, 128, 128, BF16, bad) == ctypes.c_size_t(-1).value
    assert _ws(lib, 1, 64, 1, 128, 128, BF16, K_.Plan(1, 64, 3)) == 0
    # state snapshots come from the chunk state pass: not with the token-serial form
    assert _snap(lib, dt=F32) == UNSUPPORTED
    assert _snap(lib, dt=F32, K=64, V=64, ws=None) == WORKSPACE  # supported: fails only on the workspace


def test_prefill_rejects_null_and_misaligned_pointers():
    lib = _lib()
    for name in ("q", "k", "v", "g", "beta", "o"):
        assert _fwd(lib, **{name: None}) == INVALID, name
    for name in ("q", "k", "v", "g", "o"):
        assert _fwd(lib, **{name: FAKE + 2}) == INVALID, name
    assert _fwd(lib, beta=FAKE + 1) == INVALID
    assert _fwd(lib, dt=F32, K=64, V=64, beta=FAKE + 2) == INVALID
    assert _fwd(lib, s0=FAKE + 4) == INVALID
    assert _fwd(lib, sT=FAKE + 8) == INVALID


def test_prefill_rejects_partially_overlapping_states():
    lib = _lib()
    # B*H*K*V*4 bytes per state; offset by 16 bytes: partial overlap
    assert _fwd(lib, s0=FAKE, sT=FAKE + 16) == INVALID


def test_prefill_workspace_check_with_explicit_plan():
    lib = _lib()
    T, H = 64 * 40, 2
    seg = (3 * 2 * 128 * 256 + 2 * 128 * 128) * 4     # (n_seg-1) B H K (K+V) + B H K V fp32 words
    # one record per (b, h, chunk): W, Qh [64 x 128], Mqk [64 x 64], KbT, UtT [128 x 64] bf16, e^{G_C} fp32
    rec = 2 * (64 * 128 * 2 + 64 * 64 + 2 * 128 * 64) + 128 * 4
    assert rec % 256 == 0
    for plan, need_expected in ((K_.Plan(4, 64, 1), seg), (K_.Plan(4, 64, 2), seg + H * 40 * rec),
                                (K_.Plan(1, 64, 2), H * 40 * rec), (K_.Plan(1, 128, 1), 0)):
        need = _ws(lib, 1, T, H, 128, 128, BF16, plan)
        assert need == need_expected, (plan.n_seg, plan.v_block, plan.split)
        if need:
            assert _fwd(lib, T=T, H=H, plan=plan, ws=None) == WORKSPACE
            assert _fwd(lib, T=T, H=H, plan=plan, ws=FAKE, ws_bytes=need - 1) == WORKSPACE


def test_noalloc_validates_before_taking_its_scratch():
    # host checks and the plan choice come before any HIP call; an explicit
    # plan whose workspace exceeds the 64 MiB scratch array is rejected
    lib = _lib()
    p = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(B=1, T=64, H=1, K=128, V=128, dt=BF16, q=FAKE, s0=None, sT=None, plan=None):
        return lib.kda_chunk_fwd_noalloc(B, T, H, K, V, dt, p(q), p(FAKE), p(FAKE), p(FAKE), p(FAKE), p(s0),
                                         p(FAKE), p(sT), None if plan is None else ctypes.byref(plan), None)
    assert call(K=96) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(q=None) == INVALID
    assert call(s0=FAKE, sT=FAKE + 16) == INVALID
    # 16 segments of 64 (b, h) chains: 15 * 64 * 128 KiB of transitions and
    # local states plus 4 MiB, above 64 MiB; records of the two-pass plan too
    big = dict(B=1, T=64 * 160, H=64)
    assert _ws(lib, 1, 64 * 160, 64, 128, 128, BF16, K_.Plan(16, 128, 1)) == (15 * 64 + 64) * 128 * 128 * 4 + \
        15 * 64 * 128 * 128 * 4
    assert _ws(lib, 1, 64 * 160, 64, 128, 128, BF16, K_.Plan(16, 128, 1)) > K_.NOALLOC_SCRATCH_BYTES
    assert call(plan=K_.Plan(16, 128, 1), **big) == WORKSPACE
    assert call(plan=K_.Plan(1, 128, 2), **big) == WORKSPACE
    assert call(B=0, q=None) == OK                   # nothing to do, no scratch taken
    assert call(H=0, q=None) == OK


def test_prefill_rejects_bad_plans():
    lib = _lib()
    assert _fwd(lib, plan=K_.Plan(1, 96)) == INVALID
    assert _fwd(lib, plan=K_.Plan(-1, 64)) == INVALID
    assert _fwd(lib, K=64, V=64, plan=K_.Plan(1, 128)) == UNSUPPORTED
    # a segmented plan needs value blocks that tile the K transition columns
    assert _fwd(lib, T=64 * 40, K=64, V=128, plan=K_.Plan(2, 128), ws=FAKE, ws_bytes=1 << 30) == UNSUPPORTED
    assert _fwd(lib, plan=K_.Plan(1, 64, 5)) == INVALID
    # the fused plan holds every value column of bf16 K = V = 128 in one workgroup
    assert _fwd(lib, plan=K_.Plan(1, 64, 4)) == UNSUPPORTED
    assert _fwd(lib, K=64, V=64, plan=K_.Plan(1, 0, 4)) == UNSUPPORTED
    assert _fwd(lib, dt=F32, plan=K_.Plan(1, 0, 4)) == UNSUPPORTED
    assert _fwd(lib, plan=K_.Plan(1, 64, -1)) == INVALID
    bad = K_.Plan(1, 96)
    assert _ws(lib, 1, 64, 1, 128, 128, BF16, bad) == ctypes.c_size_t(-1).value


def test_prefill_empty_batch_is_a_no_op():
    lib = _lib()
    assert _fwd(lib, B=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK
    assert _fwd(lib, H=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def test_decode_rejects_bad_arguments():
    lib = _lib()
    p = ctypes.c_void_p
    args = lambda **kw: [kw.get(n, p(FAKE)) for n in ("q", "k", "v", "g", "beta", "state", "o")]
    assert lib.kda_recurrent_step(-1, 1, 128, 128, BF16, *args(), None) == INVALID
    assert lib.kda_recurrent_step(1, 1, 100, 128, BF16, *args(), None) == UNSUPPORTED
    assert lib.kda_recurrent_step(1, 1, 128, 128, 5, *args(), None) == INVALID
    for name in ("q", "k", "v", "g", "beta", "state", "o"):
        assert lib.kda_recurrent_step(2, 2, 128, 128, BF16, *args(**{name: None}), None) == INVALID, name
    assert lib.kda_recurrent_step(2, 2, 128, 128, BF16, *args(state=p(FAKE + 4)), None) == INVALID
    assert lib.kda_recurrent_step(0, 2, 128, 128, BF16, *args(), None) == OK


def test_profile_calls_validate_without_a_gpu():
    lib = _lib()
    lib.kda_profile_stop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.kda_profile_stop.restype = ctypes.c_int
    assert lib.kda_profile_stop(None, None, 0) == -1          # never started
    assert lib.kda_profile_start(0) == INVALID
    assert lib.kda_profile_start(-3) == INVALID
    assert lib.kda_profile_start((1 << 20) + 1) == INVALID


def _varlen(lib, N=3, cu=FAKE, T=300, H=2, K=128, V=128, dt=BF16, s0=None, sT=None, ws=FAKE, ws_bytes=1 << 40,
            **kw):
    p = ctypes.c_void_p
    t = {n: kw.get(n, FAKE) for n in ("q", "k", "v", "g", "beta", "o")}
    return lib.kda_chunk_fwd_varlen(N, p(cu) if cu else None, T, H, K, V, dt, *(p(t[n]) if t[n] else None for n in
                                    ("q", "k", "v", "g", "beta")), p(s0) if s0 else None,
                                    p(t["o"]) if t["o"] else None, p(sT) if sT else None, p(ws) if ws else None,
                                    ws_bytes, None)


def test_varlen_validation_before_any_launch():
    lib = _lib()
    assert _varlen(lib, N=-1) == INVALID
    assert _varlen(lib, cu=None) == INVALID
    assert _varlen(lib, cu=FAKE + 2) == INVALID                  # int32 alignment
    assert _varlen(lib, K=96) == UNSUPPORTED
    assert _varlen(lib, q=None) == INVALID
    assert _varlen(lib, o=FAKE + 8) == INVALID
    assert _varlen(lib, s0=FAKE, sT=FAKE + 16) == INVALID        # partial state overlap
    assert _varlen(lib, ws=None) == WORKSPACE
    assert _varlen(lib, N=0) == OK                               # nothing to do
    assert _varlen(lib, H=0) == OK


def test_varlen_workspace_formula():
    lib = _lib()
    N, T, H = 5, 1000, 3
    rec = 2 * (64 * 128 * 2 + 64 * 64 + 2 * 128 * 64) + 128 * 4
    bound = -(-T // 64) + N                  # sum_i ceil(len_i / 64) <= ceil(T / 64) + N
    offs = -(-(N + 1) * 4 // 256) * 256      # chunk offsets, then snapshot offsets
    assert lib.kda_chunk_fwd_varlen_workspace_size(N, T, H, 128, 128, BF16) == 2 * offs + H * bound * rec
    assert lib.kda_chunk_fwd_varlen_workspace_size(-1, T, H, 128, 128, BF16) == ctypes.c_size_t(-1).value
    assert _varlen(lib, N=N, T=T, H=H, ws_bytes=2 * offs + H * bound * rec - 1) == WORKSPACE


def _snap(lib, interval=128, snaps=FAKE, cap=4, N=3, T=300, H=2, K=128, V=128, ws=FAKE, ws_bytes=1 << 40,
          dt=BF16):
    p = ctypes.c_void_p
    lib.kda_chunk_fwd_varlen_snapshots.argtypes = [ctypes.c_int, p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int] + [p] * 8 + \
        [ctypes.c_int, p, ctypes.c_int, p, ctypes.c_size_t, p]
    lib.kda_chunk_fwd_varlen_snapshots.restype = ctypes.c_int
    return lib.kda_chunk_fwd_varlen_snapshots(N, p(FAKE), T, H, K, V, dt, *([p(FAKE)] * 5), None, p(FAKE), None,
                                              interval, p(snaps) if snaps else None, cap, p(ws) if ws else None,
                                              ws_bytes, None)


def test_varlen_snapshot_validation_before_any_launch():
    lib = _lib()
    assert _snap(lib, interval=0) == INVALID                     # snapshots need an interval
    assert _snap(lib, interval=-64) == INVALID
    assert _snap(lib, interval=100) == INVALID                   # not a multiple of the chunk
    assert _snap(lib, snaps=None) == INVALID                     # capacity without a buffer
    assert _snap(lib, snaps=FAKE + 8) == INVALID                 # 16-byte alignment
    assert _snap(lib, cap=-1) == INVALID
    assert _snap(lib, K=96) == UNSUPPORTED
    assert _snap(lib, ws=None) == WORKSPACE
    assert _snap(lib, N=0) == OK                                 # nothing to do
    assert _snap(lib, snaps=None, cap=0, N=0) == OK


def test_snapshot_count_formula():
    # sum_i floor(len_i / interval) over the packed lengths
    assert K_.snapshot_count([0, 64, 64, 300, 1000], 128) == 0 + 0 + 1 + 5
    assert K_.snapshot_count([0], 64) == 0
    assert K_.snapshot_count([0, 640], 64) == 10


def _steps(lib, N=2, T=3, H=2, K=128, V=128, dt=BF16, state=FAKE, steps=None, **kw):
    p = ctypes.c_void_p
    lib.kda_recurrent_steps.argtypes = [ctypes.c_int] * 6 + [p] * 9
    lib.kda_recurrent_steps.restype = ctypes.c_int
    t = {n: kw.get(n, FAKE) for n in ("q", "k", "v", "g", "beta", "o")}
    return lib.kda_recurrent_steps(N, T, H, K, V, dt, *(p(t[n]) if t[n] else None for n in ("q", "k", "v", "g", "beta")),
                                   p(state) if state else None, p(t["o"]) if t["o"] else None,
                                   p(steps) if steps else None, None)


def test_recurrent_steps_validation_before_any_launch():
    lib = _lib()
    assert _steps(lib, T=-1) == INVALID
    assert _steps(lib, N=-1) == INVALID
    assert _steps(lib, K=96) == UNSUPPORTED
    assert _steps(lib, dt=7) == INVALID
    assert _steps(lib, state=None) == INVALID
    assert _steps(lib, state=FAKE + 4) == INVALID                 # 16-byte alignment
    assert _steps(lib, q=FAKE + 1) == INVALID                     # element alignment
    assert _steps(lib, steps=FAKE + 8) == INVALID                 # 16-byte alignment
    # step states may not share a byte with the state
    nbytes = 2 * 2 * 128 * 128 * 4
    assert _steps(lib, steps=FAKE) == INVALID
    assert _steps(lib, steps=FAKE + nbytes - 16) == INVALID
    assert _steps(lib, steps=FAKE - 3 * nbytes + 16) == INVALID
    assert _steps(lib, T=0) == OK                                 # nothing to do
    assert _steps(lib, N=0) == OK


def test_gated_entry_points_validate_the_gate():
    lib = _lib()
    p = ctypes.c_void_p
    lib.kda_chunk_fwd_gated.argtypes = [ctypes.c_int] * 6 + [p] * 9 + [p, p, ctypes.c_size_t, p]
    lib.kda_chunk_fwd_gated.restype = ctypes.c_int
    args = lambda gate: (1, 100, 2, 128, 128, BF16, *([p(FAKE)] * 5), p(gate) if gate else None, None,
                         p(FAKE), None, None, p(FAKE), 1 << 40, None)
    assert lib.kda_chunk_fwd_gated(*args(None)) == INVALID         # a gated call needs the gate
    assert lib.kda_chunk_fwd_gated(*args(FAKE + 8)) == INVALID     # 16-byte alignment
    lib.kda_chunk_fwd_varlen_gated.argtypes = [ctypes.c_int, p] + [ctypes.c_int] * 5 + [p] * 9 + \
        [p, ctypes.c_size_t, p]
    lib.kda_chunk_fwd_varlen_gated.restype = ctypes.c_int
    vargs = lambda gate, N=3: (N, p(FAKE), 300, 2, 128, 128, BF16, *([p(FAKE)] * 5),
                               p(gate) if gate else None, None, p(FAKE), None, p(FAKE), 1 << 40, None)
    assert lib.kda_chunk_fwd_varlen_gated(*vargs(None)) == INVALID
    assert lib.kda_chunk_fwd_varlen_gated(*vargs(FAKE + 4)) == INVALID
    assert lib.kda_chunk_fwd_varlen_gated(*vargs(None, N=0)) == OK   # nothing to do


def _bwd(lib, B=1, T=100, H=2, K=128, V=128, dt=BF16, ws=FAKE, ws_bytes=1 << 40, ds0=None, dsT=None, **kw):
    p = ctypes.c_void_p
    lib.kda_chunk_bwd.argtypes = [ctypes.c_int] * 6 + [p] * 14 + [p, ctypes.c_size_t, p]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    t = {n: kw.get(n, FAKE) for n in ("q", "k", "v", "g", "beta", "do", "dq", "dk", "dv", "dg", "dbeta")}
    pt = lambda n: p(t[n]) if t[n] else None
    return lib.kda_chunk_bwd(B, T, H, K, V, dt, pt("q"), pt("k"), pt("v"), pt("g"), pt("beta"), None, pt("do"),
                             p(dsT) if dsT else None,
                             pt("dq"), pt("dk"), pt("dv"), pt("dg"), pt("dbeta"), p(ds0) if ds0 else None,
                             p(ws) if ws else None, ws_bytes, None)


def test_backward_validation_before_any_launch():
    lib = _lib()
    assert _bwd(lib, K=96) == UNSUPPORTED
    assert _bwd(lib, T=-1) == INVALID
    assert _bwd(lib, dt=5) == INVALID
    assert _bwd(lib, dq=None) == INVALID
    assert _bwd(lib, dbeta=None) == INVALID
    assert _bwd(lib, dv=FAKE + 1) == INVALID                    # element alignment
    assert _bwd(lib, ds0=FAKE + 8) == INVALID                   # 16-byte alignment
    assert _bwd(lib, ws=None) == WORKSPACE
    assert _bwd(lib, B=0) == OK
    # dL/dS_0 may not share a byte with dL/dS_T (read and written by the same
    # reverse pass): exact alias and partial overlap are both rejected
    nstate = 2 * 128 * 128 * 4
    assert _bwd(lib, ds0=FAKE, dsT=FAKE) == INVALID
    assert _bwd(lib, ds0=FAKE + nstate - 16, dsT=FAKE) == INVALID
    assert _bwd(lib, ds0=FAKE, dsT=FAKE + nstate - 16) == INVALID
    assert _bwd(lib, ds0=FAKE, dsT=FAKE + nstate, ws=None) == WORKSPACE   # disjoint: passes the check
    lib.kda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    ck = -(-(2 * 13 * 128 * 128 * 4) // 256) * 256              # the state every 8 tokens
    tok = ck + 8 * (100 * 2) * (3 * 128 + 1) * 4                # partial sums per 16-column block
    # whole-sequence schedule (fp32 at K = V = 128): checkpoints and partial sums
    assert lib.kda_chunk_bwd_workspace_size(1, 100, 2, 128, 128, F32) == tok
    # chunk form: 2 chunks of 2 (b, h) chains, one segment: the chunk records
    # (W, Qh, Mqk, KbT, U~^T bf16; e^{G_C} fp32), the state after every chunk
    # and dL/dS after every chunk, then per chunk the fp32 dU of the reverse
    # pass.  bf16 at K = V = 128 computes every gradient of a chunk in one
    # workgroup and keeps nothing else; its states and adjoints are bf16, and
    # it keeps bf16 copies of S0 and dL/dS_T
    n = lib.kda_chunk_bwd_workspace_size(1, 100, 2, 128, 128, BF16)
    rec = (64 * 128 * 2 * 4 + 64 * 64 * 2 + 128 * 4 + 255) // 256 * 256
    assert n == 4 * rec + 2 * (4 * 128 * 128 * 2) + 4 * (64 * 128) * 4 + 2 * (2 * 128 * 128 * 2)
    # the three-stage form (here K = 128, V = 64) keeps per chunk dU, D, dQh,
    # dKb, dW, rs, dKh, Et
    n64 = lib.kda_chunk_bwd_workspace_size(1, 100, 2, 128, 64, BF16)
    rec64 = (64 * 128 * 2 * 3 + 64 * 64 * 2 + 64 * 64 * 2 + 128 * 4 + 255) // 256 * 256
    inter = 64 * 64 + 64 * 64 + 4 * 64 * 128 + 128 + 64 * 64
    assert n64 == 4 * rec64 + 2 * (4 * 128 * 64 * 4) + 4 * inter * 4
    assert _bwd(lib, ws_bytes=n - 1) == WORKSPACE
    assert lib.kda_chunk_bwd_workspace_size(1, 0, 2, 128, 128, BF16) == 0
    # several segments (40 chunks of 2 chains, planned for 256 CUs: 10
    # segments of 4 chunks): the segment arrays hold the transitions of all
    # 10 segments (the reverse scan applies their transposes) and the loads
    n10 = lib.kda_chunk_bwd_workspace_size(1, 64 * 40, 2, 128, 128, BF16)
    seg = -(-((10 * 2 * 128 * 128 + 10 * 2 * 128 * 128) * 4) // 256) * 256
    assert n10 == (seg + 2 * 40 * rec + 2 * (2 * 40 * 128 * 128 * 2) + 2 * 40 * (64 * 128) * 4
                   + 2 * (2 * 128 * 128 * 2))


def test_package_raises_without_library(tmp_path):
    saved = K_._lib
    K_._lib = None
    try:
        with pytest.raises(RuntimeError):
            K_.load_library(str(tmp_path / "missing.so"))
    finally:
        K_._lib = saved
