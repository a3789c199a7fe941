"""GPU parity of the token-serial prefill: the form the library takes for
fp32 inputs with K = 128 (no chunk kernel fits those sizes), and on request
(plan split = 3) for any supported size.  Every result is checked against the
fp64 oracle; fp32 K = 64, V = 128 (single-pass chunk kernel in 64-column
blocks; the packed batch takes the token-serial form) is covered alongside."""
import numpy as np
import pytest
import torch

from gated_delta_rule_66_amd import chunk_fwd, chunk_fwd_varlen, chunk_plan
from gated_delta_rule_66_amd.inputs import make_prefill
from tests.parity import TOL, o_err, s_err
from tests.test_gpu_parity import DEV, _gate, _gate_close, _packed, gpu_fwd, run_oracle, say, to_dev

pytestmark = pytest.mark.gpu
F32 = torch.float32


@pytest.mark.parametrize("B,T,H,K,V", [(1, 200, 2, 128, 128), (2, 77, 3, 128, 64), (2, 150, 2, 64, 128),
                                       (1, 1, 1, 128, 128), (1, 64, 2, 128, 128)])
def test_fp32_wide_prefill_matches_oracle(B, T, H, K, V):
    say("fp32 prefill B=%d T=%d H=%d K=%d V=%d" % (B, T, H, K, V))
    if K == 128:
        assert chunk_plan(B, T, H, K, V, F32) == (1, 64, 3)
    d = make_prefill(B, T, H, K, V, F32, seed=300 + T, s0_std=0.02)
    o, sT = gpu_fwd(to_dev(d))
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[F32]
    assert s_err(sT, s_ref) < TOL[F32]


def test_fp32_wide_zero_state_and_in_place_resume():
    """No initial state (zeros); and a final state written over the initial
    one equals the separate-buffer result bit for bit."""
    say("fp32 K=V=128: no S0; in-place resume")
    d = make_prefill(2, 90, 2, 128, 128, F32, seed=311, s0_std=None)
    x = to_dev(d)
    o, sT = gpu_fwd(x)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[F32] and s_err(sT, s_ref) < TOL[F32]
    d = make_prefill(2, 90, 2, 128, 128, F32, seed=312, s0_std=0.02)
    x = to_dev(d)
    o1, s1 = gpu_fwd(x)
    state = x["s0"].clone()
    o2, s2 = chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], state, True, None, final_state=state)
    torch.cuda.synchronize()
    assert s2.data_ptr() == state.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, state)


def test_fp32_wide_output_gate():
    say("fp32 K=V=128 with the output gate")
    d = make_prefill(2, 120, 2, 128, 128, F32, seed=320, s0_std=0.02)
    z = _gate((2, 120, 2, 128), F32, seed=321)
    x = to_dev(d)
    zd = z.to(DEV)
    o_plain, s_plain = gpu_fwd(x)
    o_gated, s_gated = gpu_fwd(x, gate=zd)
    torch.cuda.synchronize()
    assert torch.equal(s_gated, s_plain)
    assert _gate_close(o_gated, o_plain, zd, F32)
    o_ref, _ = run_oracle(d)
    g_ref = np.asarray(o_ref, np.float64) / (1.0 + np.exp(-z.double().numpy()))
    assert o_err(o_gated, g_ref) < TOL[F32]


@pytest.mark.parametrize("lengths,H,K,V", [([0, 1, 63, 200, 5], 2, 128, 128), ([33, 0, 130], 3, 64, 128),
                                           ([64, 100], 2, 128, 64)])
def test_fp32_wide_packed_batch(lengths, H, K, V):
    """A packed fp32 batch equals the oracle per sequence and one call per
    sequence bit for bit (both token-serial)."""
    say("fp32 varlen lengths=%s H=%d K=%d V=%d" % (lengths, H, K, V))
    seqs, x, cu = _packed(lengths, H, K, V, F32, seed=330)
    xd = to_dev(x)
    o, sT = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cu.to(DEV), xd["s0"])
    torch.cuda.synchronize()
    for i, (d, n) in enumerate(zip(seqs, lengths)):
        a, e = int(cu[i]), int(cu[i + 1])
        o_ref, s_ref = run_oracle(d)
        if n:
            assert o_err(o[a:e][None], o_ref) < TOL[F32], i
        assert s_err(sT[i:i + 1], s_ref) < TOL[F32], i
        if n and K == 128:
            o1, s1 = gpu_fwd(to_dev(d))
            torch.cuda.synchronize()
            assert torch.equal(o[a:e], o1[0]) and torch.equal(sT[i:i + 1], s1), i


def test_fp32_wide_packed_batch_gate():
    say("fp32 varlen with the output gate")
    seqs, x, cu = _packed([50, 0, 77], 2, 128, 128, F32, seed=340)
    xd = to_dev(x)
    z = _gate((int(cu[-1]), 2, 128), F32, seed=341).to(DEV)
    cud = cu.to(DEV)
    o_plain, s_plain = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"])
    o_gated, s_gated = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"], gate=z)
    torch.cuda.synchronize()
    assert torch.equal(s_gated, s_plain)
    assert _gate_close(o_gated, o_plain, z, F32)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_token_form_on_request_bf16(K, V):
    """The token-serial form requested for bf16 inputs: against the oracle
    at the bf16 tolerance."""
    say("token form bf16 K=%d V=%d" % (K, V))
    d = make_prefill(2, 140, 2, K, V, torch.bfloat16, seed=350, s0_std=0.02)
    o, sT = gpu_fwd(to_dev(d), (1, 64, 3))
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[torch.bfloat16]
    assert s_err(sT, s_ref) < TOL[torch.bfloat16]
