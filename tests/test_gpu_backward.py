"""GPU parity of the backward (``kda_chunk_bwd``, through the C ABI) against
the oracle's backward: every gradient, per (b, h) chain, as relative L2."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_66_amd import chunk_bwd
from gated_delta_rule_66_amd.inputs import make_prefill
from tests.parity import TOL, max_rel_l2

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print("[case] " + msg, flush=True)


def _grads_in(B, T, H, K, V, dtype, seed, with_s0=True, with_dst=True):
    d = make_prefill(B, T, H, K, V, dtype, seed=seed, s0_std=0.02 if with_s0 else None)
    gen = torch.Generator().manual_seed(seed + 1000)
    d_o = torch.randn((B, T, H, V), generator=gen).to(dtype)
    dsT = torch.randn((B, H, K, V), generator=gen) if with_dst else None
    return d, d_o, dsT


def _check(dq, dk, dv, dg, db, ds0, ref, dtype):
    rq, rk, rv, rg, rb, rs = ref
    tol = TOL[dtype]
    assert max_rel_l2(dq, rq, (0, 2)) < tol, "dq"
    assert max_rel_l2(dk, rk, (0, 2)) < tol, "dk"
    assert max_rel_l2(dv, rv, (0, 2)) < tol, "dv"
    assert max_rel_l2(dg, rg, (0, 2)) < tol, "dg"
    assert max_rel_l2(db, rb, (0, 2)) < tol, "dbeta"
    if ds0 is not None:
        assert max_rel_l2(ds0, rs, (0, 1)) < tol, "ds0"


# the last four run the reverse state pass over several segments (10, 4, 11
# and 78 segments of the plan for a 256-CU device)
CASES = [(2, 1, 2, 128, 128, torch.bfloat16), (1, 7, 2, 64, 64, torch.float32),
         (2, 9, 2, 128, 64, torch.bfloat16), (1, 100, 3, 64, 128, torch.bfloat16),
         (2, 300, 2, 128, 128, torch.bfloat16), (1, 257, 2, 128, 128, torch.float32),
         (1, 2597, 2, 128, 128, torch.bfloat16), (1, 1100, 1, 64, 64, torch.float32),
         (1, 3000, 1, 64, 64, torch.bfloat16), (1, 20000, 1, 128, 128, torch.bfloat16)]


@pytest.mark.parametrize("B,T,H,K,V,dtype", CASES)
def test_backward_matches_oracle(B, T, H, K, V, dtype):
    say("bwd B=%d T=%d H=%d K=%d V=%d %s" % (B, T, H, K, V, dtype))
    d, d_o, dsT = _grads_in(B, T, H, K, V, dtype, seed=90 + T)
    x = {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    out = chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o.to(DEV), dsT.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.oracle_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d_o, dsT)
    _check(*out, ref, dtype)


def test_backward_with_floor_channels():
    """A quarter of the (head, channel) pairs hold g = -5 (the clamp floor) at
    every token: the largest in-block exponents (16 tokens at the floor) and
    the gate derivative on the closed end of the clamp range."""
    say("bwd: 25 % floor channels, B=2 T=300 H=2 K=V=128 bf16")
    d = make_prefill(2, 300, 2, 128, 128, torch.bfloat16, seed=97, s0_std=0.02, pinned_frac=0.25)
    gen = torch.Generator().manual_seed(1097)
    d_o = torch.randn((2, 300, 2, 128), generator=gen).to(torch.bfloat16)
    dsT = torch.randn((2, 2, 128, 128), generator=gen)
    x = {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    out = chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o.to(DEV), dsT.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.oracle_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d_o, dsT)
    _check(*out, ref, torch.bfloat16)


def test_backward_without_incoming_state_gradient_or_initial_state():
    say("bwd: no S0, no dS_T, no dS0 output")
    d, d_o, _ = _grads_in(2, 130, 2, 128, 128, torch.bfloat16, seed=95, with_s0=False, with_dst=False)
    x = {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
    out = chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, d_o.to(DEV), None,
                    want_d_initial_state=False)
    torch.cuda.synchronize()
    assert out[5] is None
    ref = oracle.oracle_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d_o, None)
    _check(*out[:5], None, ref, torch.bfloat16)


def test_backward_deterministic_and_t0():
    say("bwd: bitwise repeat (three chunk stages at K = V = 64, one fused kernel at 128); T = 0")
    for K, T in ((64, 70), (128, 200)):
        d, d_o, dsT = _grads_in(1, T, 2, K, K, torch.bfloat16, seed=96)
        x = {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in d.items()}
        a = chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o.to(DEV), dsT.to(DEV))
        b = chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o.to(DEV), dsT.to(DEV))
        torch.cuda.synchronize()
        for u, w in zip(a, b):
            assert torch.equal(u, w)
    z = {n: t[:, :0].contiguous() for n, t in x.items() if n != "s0"}
    dsT_d = dsT.to(DEV)
    out = chunk_bwd(z["q"], z["k"], z["v"], z["g"], z["beta"], x["s0"], None, dsT_d)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dsT_d)          # no tokens: dL/dS_0 = dL/dS_T


def test_backward_full_8k_workload_sampled():
    """The 8K workload (B=1, T=8192, H=32, K=V=128 bf16) as bench.py times
    it: all gradients of sampled (b, h) chains against the oracle."""
    from gated_delta_rule_66_amd.inputs import CONFIGS, make_prefill_config
    say("bwd full 8K workload, sampled chains")
    c = CONFIGS["prefill_8k"]
    x = make_prefill_config(c, "cpu")
    B, T, H, K, V = c.B, c.T, c.H, c.K, c.V
    gen = torch.Generator().manual_seed(12)
    d_o = torch.randn((B, T, H, V), generator=gen).to(c.dtype)
    xd = {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in x.items()}
    out = chunk_bwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["s0"], d_o.to(DEV), None)
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    sl = lambda t: t[:, :, heads].contiguous()          # the sampled chains side by side (oracle threads)
    s0 = None if x["s0"] is None else x["s0"][:, heads].contiguous()
    ref = oracle.oracle_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), s0, sl(d_o), None)
    got = [sl(t.cpu()) for t in out[:5]] + [out[5][:, heads].cpu()]
    _check(*got, ref, c.dtype)
