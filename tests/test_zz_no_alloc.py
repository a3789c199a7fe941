"""kda_chunk_fwd_noalloc (workspace in the library's per-GPU scratch array)
against kda_chunk_fwd / kda_chunk_fwd_planned in the same plan, through the
C ABI, on calls in a row of shrinking size.  The two entry points run the same
kernels in the same plan, so their results are compared bit for bit (which
implies the parity bar of the planned call)."""
import pytest
import torch

import gated_delta_rule_66_amd as kda
from gated_delta_rule_66_amd.inputs import make_prefill
from tests.parity import TOL, o_err, s_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print("[case] " + msg, flush=True)


def _inputs(B, T, H, seed, s0, K=128, V=128):
    d = make_prefill(B, T, H, K, V, torch.bfloat16, seed=seed, s0_std=0.02 if s0 else None)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _reference_plan(B, T, H, K=128, V=128):
    """The plan the no-alloc call runs when left to the library: the library's
    plan if its workspace fits the scratch array, else the single pass with
    the library's segment count (smaller if needed)."""
    ws = kda.chunk_workspace_size(B, T, H, K, V, torch.bfloat16)
    if ws <= kda.kda.NOALLOC_SCRATCH_BYTES:
        return None
    plan = (0, 0, 1)
    assert kda.chunk_workspace_size(B, T, H, K, V, torch.bfloat16, plan) <= kda.kda.NOALLOC_SCRATCH_BYTES
    return plan


def _compare(x, plan, in_place):
    B, T, H, K = x["q"].shape
    V = x["v"].shape[-1]
    ref_plan = plan if plan is not None else _reference_plan(B, T, H, K, V)
    o_ref = torch.empty_like(x["v"])
    o_na = torch.full_like(x["v"], float("nan"))
    if in_place:
        s_ref = x["s0"].clone()
        s_na = x["s0"].clone()
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s_ref, True, ref_plan, out=o_ref,
                      final_state=s_ref)
        kda.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], s_na, out=o_na, final_state=s_na,
                              plan=plan)
    else:
        s_ref = torch.empty((B, H, K, V), dtype=torch.float32, device=DEV)
        s_na = torch.full_like(s_ref, float("nan"))
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], True, ref_plan, out=o_ref,
                      final_state=s_ref)
        kda.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], out=o_na, final_state=s_na,
                              plan=plan)
    torch.cuda.synchronize()
    assert o_err(o_na, o_ref) < TOL[torch.bfloat16]
    assert s_err(s_na, s_ref) < TOL[torch.bfloat16]
    assert torch.equal(o_na, o_ref) and torch.equal(s_na, s_ref)


def test_noalloc_matches_the_planned_call_on_shrinking_inputs():
    # 1) K = V = 64: the library's two-pass plan would need more than 64 MiB
    #    of records, so the no-alloc call runs the segmented single pass
    say("noalloc: B=1 T=13440 H=8 K=V=64, library plan left to the bound")
    x = _inputs(1, 64 * 210, 8, seed=41, s0=True, K=64, V=64)
    assert kda.chunk_workspace_size(1, 64 * 210, 8, 64, 64, torch.bfloat16) > kda.kda.NOALLOC_SCRATCH_BYTES
    assert _reference_plan(1, 64 * 210, 8, 64, 64) == (0, 0, 1)
    _compare(x, None, in_place=False)
    # 1b) K = V = 128: the library's fused plan, its segment arrays in the scratch
    say("noalloc: B=1 T=2560 H=4, the library's segmented plan")
    w = _inputs(1, 64 * 40, 4, seed=46, s0=True)
    assert _reference_plan(1, 64 * 40, 4) is None
    assert kda.chunk_plan(1, 64 * 40, 4, 128, 128, torch.bfloat16)[0] > 1
    _compare(w, None, in_place=True)
    # 2) smaller, an explicit segmented plan, final state in place over the
    #    initial state (the redirected final state also sits in the scratch)
    say("noalloc: B=1 T=323 H=2, plan (3, 64, 1), in place")
    y = _inputs(1, 64 * 5 + 3, 2, seed=42, s0=True)
    _compare(y, (3, 64, 1), in_place=True)
    # 3) smaller still, the library's own plan (its records fit the scratch)
    say("noalloc: B=2 T=100 H=2, library plan")
    z = _inputs(2, 100, 2, seed=43, s0=False)
    assert _reference_plan(2, 100, 2) is None
    _compare(z, None, in_place=False)
    # 4) the first input again: nothing left over from the calls between
    say("noalloc: B=1 T=13440 H=8 K=V=64 again")
    _compare(x, None, in_place=False)


def test_noalloc_empty_and_rejected():
    say("noalloc: T=0 copies the state; a plan over the bound is rejected")
    x = _inputs(2, 0, 3, seed=44, s0=True)
    o = torch.empty_like(x["v"])
    s = torch.empty((2, 3, 128, 128), dtype=torch.float32, device=DEV)
    kda.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], out=o, final_state=s)
    torch.cuda.synchronize()
    assert torch.equal(s, x["s0"])
    y = _inputs(1, 64 * 40, 64, seed=45, s0=False)
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd_noalloc(y["q"], y["k"], y["v"], y["g"], y["beta"], None, out=torch.empty_like(y["v"]),
                              plan=(1, 128, 2))
    assert e.value.status == 3
