"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every case prints its name before it touches the GPU.  Inputs are the
seeded recipes of ``gated_delta_rule_66_amd.inputs``; the oracle always sees
the exact values the GPU saw (bf16 values upcast, no re-rounding).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_66_amd import chunk_fwd, recurrent_step, chunk_plan
from gated_delta_rule_66_amd.inputs import (CONFIGS, make_decode, make_decode_config, make_prefill,
                                            make_prefill_config)
from tests.kda_bruteforce import dense_f64_chain
from tests.parity import TOL, o_err, s_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print("[case] " + msg, flush=True)


def to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_oracle(d):
    return oracle.oracle_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"])


def gpu_fwd(x, plan=None, s0="use", split=0, **kw):
    """Prefill through the C ABI; split 1 = single-pass kernel, 2 = intra-chunk
    pass + state pass, 4 = the fused producer/consumer kernel (bf16 with
    K = V = 128 only: other shapes skip; it holds all value columns, so the
    plan's column block is left to the library), 0 = the library's choice."""
    init = x["s0"] if s0 == "use" else s0
    if split == 4:
        K, V = x["q"].shape[-1], x["v"].shape[-1]
        if not fused_exists(x["q"].dtype, K, V):
            raise ValueError("the fused kernel covers bf16 with K = V = 128 only")
        plan = (0, 0, 4) if plan is None else (plan[0], 0, 4)
    elif split:
        plan = (0, 0, split) if plan is None else (plan[0], plan[1], split)
    return chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], init, True, plan, **kw)


PATHS = [1, 2, 4]
FUSED = 4


def fused_exists(dtype, K, V):
    return dtype == torch.bfloat16 and K == 128 and V == 128


def with_paths(cases, key):
    """Every case on every path, except the fused path (split 4) for the
    sizes it has no kernel for; key(case) gives the case's (dtype, K, V)."""
    out = []
    for c in cases:
        c = c if isinstance(c, tuple) else (c,)
        out += [c + (s,) for s in PATHS if s != FUSED or fused_exists(*key(c))]
    return out


# ------------------------------------------------------------------ small cases
@pytest.mark.parametrize("split", [s for s in PATHS if s != FUSED])    # fp32, K = V = 64
def test_config0_full_parity(split):
    cfg = CONFIGS["prefill_small_fp32"]
    say("small fp32 workload: B=1 H=2 T=256 K=V=64 split=%d" % split)
    d = make_prefill_config(cfg, "cpu")
    x = to_dev(d)
    o, sT = gpu_fwd(x, split=split)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[torch.float32]
    assert s_err(sT, s_ref) < TOL[torch.float32]


SHAPES = [
    # (K, V, T, B, H, with_s0, plan)
    (128, 128, 1, 2, 3, True, None),
    (128, 128, 15, 2, 3, True, None),
    (128, 128, 16, 1, 2, False, None),
    (128, 128, 17, 2, 3, True, None),
    (128, 128, 63, 1, 2, True, None),
    (128, 128, 64, 2, 3, True, None),
    (128, 128, 65, 1, 2, True, None),
    (128, 128, 130, 2, 3, True, (1, 128)),
    (128, 128, 1000, 1, 3, True, (1, 64)),
    (128, 128, 1000, 1, 3, True, (1, 128)),
    (64, 64, 1, 1, 2, True, None),
    (64, 64, 100, 2, 2, True, None),
    (64, 64, 640, 1, 2, False, (1, 64)),
    (128, 64, 300, 1, 2, True, None),
    (64, 128, 300, 1, 2, True, (1, 128)),
    (64, 128, 300, 1, 2, True, (1, 64)),
]


@pytest.mark.parametrize("K,V,T,B,H,with_s0,plan,split", with_paths(SHAPES, lambda c: (torch.bfloat16, c[0], c[1])))
def test_prefill_bf16_shapes(K, V, T, B, H, with_s0, plan, split):
    say("bf16 prefill K=%d V=%d T=%d B=%d H=%d s0=%s plan=%s split=%d" % (K, V, T, B, H, with_s0, plan, split))
    d = make_prefill(B, T, H, K, V, torch.bfloat16, seed=100 + T, s0_std=0.02 if with_s0 else None)
    x = to_dev(d)
    o, sT = gpu_fwd(x, plan, split=split)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[torch.bfloat16]
    assert s_err(sT, s_ref) < TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype,K,V,n_seg,split", with_paths(
    [(dt, K, V, n) for (dt, K, V) in [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64), (torch.float32, 64, 64)]
     for n in (2, 3, 7)], lambda c: c[:3]))
def test_segment_planner_matches_oracle(dtype, K, V, n_seg, split):
    """Segment transitions computed side by side and recombined: the result
    must not depend on the number of segments (page section on the one-card
    segment planner)."""
    T = 64 * 37 + 5
    say("segments dtype=%s K=%d V=%d n_seg=%d T=%d split=%d" % (dtype, K, V, n_seg, T, split))
    d = make_prefill(1, T, 2, K, V, dtype, seed=7, s0_std=0.02)
    x = to_dev(d)
    o_ref, s_ref = run_oracle(d)
    for vb in sorted({64, min(128, K, V)}):
        o, sT = gpu_fwd(x, (n_seg, vb), split=split)
        torch.cuda.synchronize()
        assert o_err(o, o_ref) < TOL[dtype], vb
        assert s_err(sT, s_ref) < TOL[dtype], vb


# ------------------------------------------------------------------ pins on the GPU
@pytest.mark.parametrize("plan", [(1, 64, 1), (1, 128, 1), (3, 64, 1), (1, 64, 2), (1, 128, 2), (3, 64, 2)])
def test_p1_no_forget_no_write(plan):
    say("P1 alpha=1 beta=0 plan=%s" % (plan,))
    d = make_prefill(1, 300, 2, 128, 128, torch.bfloat16, seed=11, s0_std=1.0)
    d["g"].zero_()
    d["beta"].zero_()
    x = to_dev(d)
    o, sT = gpu_fwd(x, plan)
    torch.cuda.synchronize()
    assert torch.equal(sT, x["s0"]), "state must be unchanged bit for bit"
    o_ref, _ = run_oracle(d)
    assert o_err(o, o_ref) < TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype,K,split", with_paths([(torch.bfloat16, 128), (torch.float32, 64)],
                                                     lambda c: (c[0], c[1], c[1])))
def test_p2_full_write_unit_key(dtype, K, split):
    say("P2 alpha=1 beta=1 basis keys dtype=%s split=%d" % (dtype, split))
    T, H = 200, 2
    gen = torch.Generator().manual_seed(12)
    idx = torch.randint(0, K, (1, T, H), generator=gen)
    k = torch.nn.functional.one_hot(idx, K).to(dtype)
    v = torch.randn(1, T, H, K, generator=gen).to(dtype)
    d = dict(q=k.clone(), k=k, v=v, g=torch.zeros_like(k), beta=torch.ones(1, T, H, dtype=dtype),
             s0=torch.randn(1, H, K, K, generator=gen))
    x = to_dev(d)
    o, _ = gpu_fwd(x, split=split)
    torch.cuda.synchronize()
    assert o_err(o, v) < TOL[dtype]


@pytest.mark.parametrize("split", PATHS)
def test_p3_clamp_bitwise(split):
    say("P3 clamp: g=-50 == g=-5, g=+3 == g=0, bitwise; split=%d" % split)
    d = make_prefill(2, 257, 2, 128, 128, torch.bfloat16, seed=13, s0_std=0.02)
    x = to_dev(d)
    outs = []
    for val in (-5.0, -50.0, 0.0, 3.0):
        x["g"].fill_(val)
        outs.append(gpu_fwd(x, split=split))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[2][0], outs[3][0]) and torch.equal(outs[2][1], outs[3][1])
    # mixed out-of-range channels against the oracle (the all-floor stress run)
    g = d["g"].float()
    g[..., ::2] = -9.0
    g[..., 1::2] = -5.0
    d["g"] = g.to(torch.bfloat16)
    x = to_dev(d)
    o, sT = gpu_fwd(x, split=split)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(sT).all()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[torch.bfloat16]
    assert s_err(sT, s_ref) < TOL[torch.bfloat16]


@pytest.mark.parametrize("split", [s for s in PATHS if s != FUSED])    # fp32, K = V = 64
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_p5_dense_expansion_short(T, split):
    say("P5 dense transition expansion T=%d split=%d" % (T, split))
    d = make_prefill(1, T, 1, 64, 64, torch.float32, seed=20 + T, s0_std=0.5)
    x = to_dev(d)
    o, sT = gpu_fwd(x, split=split)
    torch.cuda.synchronize()
    od, sd = dense_f64_chain(d["q"][0, :, 0].numpy(), d["k"][0, :, 0].numpy(), d["v"][0, :, 0].numpy(),
                             d["g"][0, :, 0].numpy(), d["beta"][0, :, 0].numpy(), d["s0"][0, 0].numpy())
    assert o_err(o, od[None, :, None, :]) < TOL[torch.float32]
    assert s_err(sT, sd[None, None]) < TOL[torch.float32]


@pytest.mark.parametrize("plan", [None, (2, 64), (0, 0, 1), (2, 64, 1)])
def test_p6_split_and_resume(plan):
    say("P6 split/resume plan=%s" % (plan,))
    T1, T2 = 700, 555
    d = make_prefill(1, T1 + T2, 3, 128, 128, torch.bfloat16, seed=14, s0_std=0.02)
    x = to_dev(d)
    o_full, s_full = gpu_fwd(x, plan)
    a = {k: (v[:, :T1].contiguous() if k != "s0" else v) for k, v in x.items()}
    o1, s1 = gpu_fwd(a, plan)
    b = {k: (v[:, T1:].contiguous() if k != "s0" else v) for k, v in x.items()}
    o2, s2 = gpu_fwd(b, plan, s0=s1)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    assert o_err(torch.cat([o1, o2], 1), o_ref) < TOL[torch.bfloat16]
    assert s_err(s2, s_ref) < TOL[torch.bfloat16]
    assert o_err(o_full, o_ref) < TOL[torch.bfloat16]
    assert s_err(s_full, s_ref) < TOL[torch.bfloat16]


@pytest.mark.parametrize("split", PATHS)
def test_p7_linearity(split):
    say("P7 linear in (S0, V) split=%d" % split)
    d = make_prefill(1, 333, 2, 128, 128, torch.bfloat16, seed=15, s0_std=0.05)
    x = to_dev(d)
    o, s = gpu_fwd(x, split=split)
    xa = dict(x)
    xa["v"] = torch.zeros_like(x["v"])
    oa, sa = gpu_fwd(xa, split=split)
    ob, sb = gpu_fwd(x, s0=None, split=split)
    torch.cuda.synchronize()
    assert o_err(oa.float() + ob.float(), o.float()) < TOL[torch.bfloat16]
    assert s_err(sa + sb, s) < TOL[torch.bfloat16]


def test_p8_prefill_then_decode_equals_longer_prefill():
    say("P8 prefill(T1) + decode x n == prefill(T1 + n); T=1 prefill == one decode step")
    T1, n = 190, 6
    d = make_prefill(2, T1 + n, 3, 128, 128, torch.bfloat16, seed=16, s0_std=0.02)
    x = to_dev(d)
    a = {k: (v[:, :T1].contiguous() if k != "s0" else v) for k, v in x.items()}
    o1, s = gpu_fwd(a)
    state = s.clone()
    outs = []
    for t in range(T1, T1 + n):
        outs.append(recurrent_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                                   x["v"][:, t].contiguous(), x["g"][:, t].contiguous(),
                                   x["beta"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(d)
    o_dec = torch.stack(outs, 1)
    assert o_err(torch.cat([o1, o_dec], 1), o_ref) < TOL[torch.bfloat16]
    assert s_err(state, s_ref) < TOL[torch.bfloat16]
    # one token: prefill and the decode kernel agree
    one = {k: (v[:, :1].contiguous() if k != "s0" else v) for k, v in x.items()}
    o_p, s_p = gpu_fwd(one)
    st = x["s0"].clone()
    o_d = recurrent_step(x["q"][:, 0].contiguous(), x["k"][:, 0].contiguous(), x["v"][:, 0].contiguous(),
                         x["g"][:, 0].contiguous(), x["beta"][:, 0].contiguous(), st)
    torch.cuda.synchronize()
    assert o_err(o_p, o_d[:, None]) < TOL[torch.bfloat16]
    assert s_err(s_p, st) < TOL[torch.bfloat16]


@pytest.mark.parametrize("plan", [(1, 64, 1), (4, 64, 1), (1, 64, 2), (4, 64, 2), (1, 0, 4), (2, 0, 4), (4, 0, 4)])
def test_in_place_state_resume(plan):
    """The final state written over S0.  The fused plan with segments reads S0
    in its first launch (segment 0 with output beside the summaries) and
    writes the final state in its last; (2, 0, 4) has no summaries at all."""
    say("final_state aliasing initial_state plan=%s" % (plan,))
    d = make_prefill(1, 64 * 20 + 9, 2, 128, 128, torch.bfloat16, seed=17, s0_std=0.02)
    x = to_dev(d)
    state = x["s0"].clone()
    o, s = chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], state, True, plan, final_state=state)
    torch.cuda.synchronize()
    assert s.data_ptr() == state.data_ptr()
    o_ref, s_ref = run_oracle(d)
    assert o_err(o, o_ref) < TOL[torch.bfloat16]
    assert s_err(state, s_ref) < TOL[torch.bfloat16]


def test_empty_sequence_copies_state():
    say("T=0")
    d = make_prefill(2, 0, 3, 128, 128, torch.bfloat16, seed=18, s0_std=0.02)
    x = to_dev(d)
    o, s = gpu_fwd(x)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128)
    assert torch.equal(s, x["s0"])
    _, s0 = gpu_fwd(x, s0=None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s0) == 0


def test_deterministic_repeat():
    say("bitwise repeatability")
    d = make_prefill(1, 64 * 30, 4, 128, 128, torch.bfloat16, seed=19, s0_std=0.02)
    x = to_dev(d)
    for plan in ((1, 64, 1), (3, 128, 1), (1, 64, 2), (3, 128, 2), (1, 128, 4), (3, 128, 4)):
        a = gpu_fwd(x, plan)
        b = gpu_fwd(x, plan)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype,K,V", [(torch.bfloat16, 64, 64), (torch.float32, 64, 64),
                                       (torch.bfloat16, 64, 128)])
def test_deterministic_repeat_k64(dtype, K, V):
    """Bitwise repeatability of the K = 64 variants on both plans, segmented
    and not: their diagonal-block inverses hand fp32 blocks between lanes of
    one wave through LDS, which needs the wave-level fence."""
    say("bitwise repeatability %s K=%d V=%d" % (dtype, K, V))
    d = make_prefill(2, 64 * 20 + 9, 3, K, V, dtype, seed=29, s0_std=0.02)
    x = to_dev(d)
    for split in (1, 2):
        for n_seg in (1, 4):
            plan = (n_seg, 64, split)
            ref = gpu_fwd(x, plan)
            for _ in range(3):
                again = gpu_fwd(x, plan)
                torch.cuda.synchronize()
                assert torch.equal(ref[0], again[0]) and torch.equal(ref[1], again[1]), plan


@pytest.mark.parametrize("split", PATHS)
@pytest.mark.parametrize("n_seg", [1, 3])
def test_p4_pure_decay_closed_form(split, n_seg):
    """P4 on the device: with beta = 0 the state only decays, so
    S_T = Diag(exp(sum_t clamp g_t)) S0 and o_t = (Diag(exp G_t) S0)^T q_t
    with G_t the running sum of the clamped gates, across chunk and segment
    boundaries (gates drawn past both clamp bounds)."""
    say("P4 beta=0 pure decay, T=300, split=%d n_seg=%d" % (split, n_seg))
    B, T, H, K, V = 1, 300, 2, 128, 128
    d = make_prefill(B, T, H, K, V, torch.bfloat16, seed=31, s0_std=0.02)
    gen = torch.Generator().manual_seed(32)
    # gates uniform in [-0.05, 0.05] (a slow mean decay, so that the state
    # stays alive over 300 tokens), channels 0-7 below the floor (-6 -> -5)
    # and channels 8-15 above the ceiling (0.5 -> 0)
    d["g"] = (torch.rand((B, T, H, K), generator=gen) * 0.1 - 0.05).to(torch.bfloat16)
    d["g"][..., 0:8] = -6.0
    d["g"][..., 8:16] = 0.5
    d["beta"] = torch.zeros_like(d["beta"])
    x = to_dev(d)
    o, sT = gpu_fwd(x, (n_seg, 128, split))
    torch.cuda.synchronize()
    gc = d["g"].double().clamp(-5.0, 0.0)                       # [B, T, H, K]
    G = torch.cumsum(gc, dim=1)                                 # running sums
    s0 = d["s0"].double()                                       # [B, H, K, V]
    s_ref = torch.exp(G[:, -1]).unsqueeze(-1) * s0              # [B, H, K, V]
    # o_t[v] = sum_c q_t[c] e^{G_t[c]} S0[c][v]
    o_ref = torch.einsum("bthc,bhcv->bthv", d["q"].double() * torch.exp(G), s0)
    assert o_err(o, o_ref.numpy()) < TOL[torch.bfloat16]
    assert s_err(sT, s_ref.numpy()) < TOL[torch.bfloat16]


def test_launch_profiling_names_every_launch():
    say("per-launch event timing: plain and segmented plans")
    import gated_delta_rule_66_amd as kda
    d = make_prefill(1, 64 * 12, 2, 128, 128, torch.bfloat16, seed=23)
    x = to_dev(d)
    ws = torch.empty(kda.chunk_workspace_size(1, 64 * 12, 2, 128, 128, torch.bfloat16, (3, 64, 2)),
                     dtype=torch.uint8, device=DEV)
    kda.profile_start(16)
    gpu_fwd(x, (1, 64, 1))
    gpu_fwd(x, (3, 64, 1), workspace=ws)
    gpu_fwd(x, (1, 64, 2), workspace=ws)
    gpu_fwd(x, (3, 64, 2), workspace=ws)
    gpu_fwd(x, (1, 0, 4))
    gpu_fwd(x, (3, 0, 4), workspace=ws)
    rec = kda.profile_stop(16)
    assert [n for n, _ in rec] == ["chunk_output", "chunk_summary", "segment_scan", "chunk_output",
                                   "intra_chunk", "state_output",
                                   "intra_chunk", "state_summary", "segment_scan", "state_output",
                                   "fused_output", "fused_summary", "segment_scan", "fused_output"]
    assert all(ms > 0 for _, ms in rec)
    o, _ = gpu_fwd(x, (1, 64))                 # timing is off again: results unchanged
    ref, _ = run_oracle(d)
    assert o_err(o, ref) < TOL[torch.bfloat16]


# ------------------------------------------------------------------ fused output gate
def _gate(shape, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=gen) * 2.0).to(dtype)


def _gate_close(fused, o_plain, z, dtype):
    """fused = RNE(o * sigmoid(z)) up to the sigmoid's hardware exp2 and
    reciprocal (about 1 ulp each): within one bf16 rounding step of the
    product torch forms in fp32, or a few fp32 ulp for fp32."""
    ref = (o_plain.float() * torch.sigmoid(z.float()))
    ulp = 2.0 ** -7 if dtype == torch.bfloat16 else 2.0 ** -19
    return bool(((fused.float() - ref).abs() <= ulp * ref.abs() + 1e-30).all())


@pytest.mark.parametrize("T,K,V,dtype,plan,split", with_paths([(300, 128, 128, torch.bfloat16, None),
                                                             (1000, 128, 128, torch.bfloat16, (3, 128)),
                                                             (130, 64, 128, torch.bfloat16, None),
                                                             (200, 64, 64, torch.float32, None)],
                                                            lambda c: (c[3], c[1], c[2])))
def test_output_gate_fused(split, T, K, V, dtype, plan):
    """o * sigmoid(gate) fused into the store of o: against the oracle's
    o * sigmoid(gate) and against the unfused composition on the GPU; the
    final state is untouched by the gate."""
    say("gate split=%d T=%d K=%d V=%d %s plan=%s" % (split, T, K, V, dtype, plan))
    d = make_prefill(2, T, 2, K, V, dtype, seed=70, s0_std=0.02)
    z = _gate((2, T, 2, V), dtype, seed=71)
    x = to_dev(d)
    zd = z.to(DEV)
    o_plain, s_plain = gpu_fwd(x, plan, split=split)
    o_gated, s_gated = gpu_fwd(x, plan, split=split, gate=zd)
    torch.cuda.synchronize()
    assert torch.equal(s_gated, s_plain)
    assert _gate_close(o_gated, o_plain, zd, dtype)
    o_ref, _ = run_oracle(d)
    g_ref = np.asarray(o_ref, np.float64) / (1.0 + np.exp(-z.double().numpy()))
    assert o_err(o_gated, g_ref) < TOL[dtype]


def test_output_gate_fused_varlen():
    from gated_delta_rule_66_amd import chunk_fwd_varlen
    say("gate varlen")
    seqs, x, cu = _packed([100, 0, 257, 64], 2, 128, 128, torch.bfloat16, seed=72)
    xd = to_dev(x)
    z = _gate((int(cu[-1]), 2, 128), torch.bfloat16, seed=73).to(DEV)
    cud = cu.to(DEV)
    o_plain, s_plain = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"])
    o_gated, s_gated = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"], gate=z)
    torch.cuda.synchronize()
    assert torch.equal(s_gated, s_plain)
    assert _gate_close(o_gated, o_plain, z, torch.bfloat16)


# ------------------------------------------------------------------ packed variable-length batches
def _packed(lengths, H, K, V, dtype, seed, s0_std=0.02):
    """Per-sequence inputs of the recipe, packed along the token axis."""
    seqs = [make_prefill(1, n, H, K, V, dtype, seed=seed + i, s0_std=s0_std) for i, n in enumerate(lengths)]
    cat = lambda name: torch.cat([d[name][0] for d in seqs], 0)
    packed = {n: cat(n) for n in ("q", "k", "v", "g", "beta")}
    packed["s0"] = torch.cat([d["s0"] for d in seqs], 0) if s0_std is not None else None
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    return seqs, packed, cu


VARLEN = [([0, 1, 63, 64, 65, 200, 7, 129], 3, 128, 128, torch.bfloat16),
          ([130, 0, 5, 64], 2, 64, 128, torch.bfloat16),
          ([70, 300, 1], 2, 128, 64, torch.bfloat16),
          ([17, 64, 100, 0, 3], 2, 64, 64, torch.float32)]


@pytest.mark.parametrize("lengths,H,K,V,dtype", VARLEN)
def test_varlen_matches_oracle_and_single_calls(lengths, H, K, V, dtype):
    """A packed batch equals the oracle per sequence, and equals (bit for
    bit) one prefill call per sequence on the same two-pass plan."""
    from gated_delta_rule_66_amd import chunk_fwd_varlen
    say("varlen lengths=%s H=%d K=%d V=%d %s" % (lengths, H, K, V, dtype))
    seqs, x, cu = _packed(lengths, H, K, V, dtype, seed=40)
    xd = to_dev(x)
    o, sT = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cu.to(DEV), xd["s0"])
    torch.cuda.synchronize()
    vb = 64     # few (sequence, head) chains: the library uses 64-column blocks
    for i, (d, n) in enumerate(zip(seqs, lengths)):
        a, e = int(cu[i]), int(cu[i + 1])
        o_ref, s_ref = run_oracle(d)
        if n:
            assert o_err(o[a:e][None], o_ref) < TOL[dtype], i
        assert s_err(sT[i:i + 1], s_ref) < TOL[dtype], i
        one = to_dev(d)
        o1, s1 = gpu_fwd(one, (1, vb, 2))
        torch.cuda.synchronize()
        assert torch.equal(o[a:e], o1[0]) and torch.equal(sT[i:i + 1], s1), i


SNAPSHOTS = [([0, 64, 200, 513, 128, 320, 7], 2, 128, 128, torch.bfloat16, 128),
             ([130, 256, 0, 64], 2, 64, 128, torch.bfloat16, 64),
             ([100, 300, 384], 2, 128, 64, torch.bfloat16, 192),
             ([128, 65, 256], 2, 64, 64, torch.float32, 64)]


@pytest.mark.parametrize("lengths,H,K,V,dtype,interval", SNAPSHOTS)
def test_varlen_snapshots_match_oracle_prefixes(lengths, H, K, V, dtype, interval):
    """Snapshot m of sequence i is the state after the first (m + 1) *
    interval tokens of that sequence (the oracle's final state on that
    prefix); o and the final states are bitwise those of the call without
    snapshots; a slot past the capacity is left untouched."""
    from gated_delta_rule_66_amd import chunk_fwd_varlen, snapshot_count
    say("varlen snapshots lengths=%s H=%d K=%d V=%d %s every %d" % (lengths, H, K, V, dtype, interval))
    seqs, x, cu = _packed(lengths, H, K, V, dtype, seed=60)
    xd = to_dev(x)
    cud = cu.to(DEV)
    o0, s0 = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"])
    o, sT, snaps = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"],
                                    snapshot_interval=interval)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(sT, s0)
    n_snap = snapshot_count(cu, interval)
    assert snaps.shape == (n_snap, H, K, V)
    base = 0
    for i, (d, n) in enumerate(zip(seqs, lengths)):
        for m in range(n // interval):
            t_end = (m + 1) * interval
            prefix = {name: (t if name == "s0" else t[:, :t_end].contiguous()) for name, t in d.items()}
            _, s_ref = run_oracle(prefix)
            assert s_err(snaps[base + m:base + m + 1], s_ref) < TOL[dtype], (i, m)
        base += n // interval
    assert base == n_snap
    # one slot less capacity: every slot below it as before, the next one untouched
    if n_snap > 1:
        big = torch.full((n_snap, H, K, V), 7.0, device=DEV)
        chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cud, xd["s0"],
                         snapshot_interval=interval, snapshots=big[:n_snap - 1])
        torch.cuda.synchronize()
        assert torch.equal(big[:n_snap - 1], snaps[:n_snap - 1])
        assert bool((big[n_snap - 1] == 7.0).all())


def test_varlen_in_place_and_empty():
    from gated_delta_rule_66_amd import chunk_fwd_varlen
    say("varlen: final state in place; all sequences empty")
    seqs, x, cu = _packed([100, 0, 65], 2, 128, 128, torch.bfloat16, seed=50)
    xd = to_dev(x)
    state = xd["s0"].clone()
    o, s = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cu.to(DEV), state, final_state=state)
    torch.cuda.synchronize()
    assert s.data_ptr() == state.data_ptr()
    for i, d in enumerate(seqs):
        _, s_ref = run_oracle(d)
        assert s_err(state[i:i + 1], s_ref) < TOL[torch.bfloat16], i
    # T_total = 0: every final state is its initial state
    z = {n: t[:0].contiguous() for n, t in xd.items() if n != "s0"}
    cu0 = torch.zeros(4, dtype=torch.int32, device=DEV)
    s0 = torch.randn(3, 2, 128, 128, device=DEV)
    o0, s_out = chunk_fwd_varlen(z["q"], z["k"], z["v"], z["g"], z["beta"], cu0, s0)
    torch.cuda.synchronize()
    assert o0.shape == (0, 2, 128) and torch.equal(s_out, s0)


def test_varlen_many_sequences_sampled():
    """A serving-size packed batch (64 sequences of mixed length, 32 heads)
    on the library's own plan, checked on sampled sequences."""
    from gated_delta_rule_66_amd import chunk_fwd_varlen
    gen = torch.Generator().manual_seed(60)
    lengths = torch.randint(0, 900, (64,), generator=gen).tolist()
    say("varlen 64 sequences, total %d tokens, H=32" % sum(lengths))
    seqs, x, cu = _packed(lengths, 32, 128, 128, torch.bfloat16, seed=61)
    xd = to_dev(x)
    o, sT = chunk_fwd_varlen(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], cu.to(DEV), xd["s0"])
    torch.cuda.synchronize()
    for i in (0, 17, 42, 63):
        a, e = int(cu[i]), int(cu[i + 1])
        o_ref, s_ref = run_oracle(seqs[i])
        if e > a:
            assert o_err(o[a:e][None], o_ref) < TOL[torch.bfloat16], i
        assert s_err(sT[i:i + 1], s_ref) < TOL[torch.bfloat16], i


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype,K,V", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 128),
                                       (torch.bfloat16, 128, 64), (torch.float32, 64, 64),
                                       (torch.float32, 128, 128)])
def test_decode_steps_match_oracle(dtype, K, V):
    say("decode dtype=%s K=%d V=%d" % (dtype, K, V))
    N, H, steps = 5, 3, 16
    d = make_decode(N, H, K, V, steps, dtype, seed=21)
    x = to_dev(d)
    state = x["state"].clone()
    ref_state = d["state"].double().numpy().copy()
    for t in range(steps):
        o = recurrent_step(x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t], state)
        o_ref = oracle.oracle_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], ref_state)
        torch.cuda.synchronize()
        assert max_rel(o, o_ref) < TOL[dtype], t
    assert s_err(state, ref_state) < TOL[dtype]


MULTI = [(torch.bfloat16, 128, 128, 4), (torch.bfloat16, 64, 128, 9), (torch.bfloat16, 128, 64, 1),
         (torch.float32, 64, 64, 5)]


@pytest.mark.parametrize("dtype,K,V,T", MULTI)
def test_multi_token_steps(dtype, K, V, T):
    """T tokens per sequence in one call: o, the final state and every
    per-token state match the oracle, and equal (bit for bit) T successive
    single decode steps."""
    from gated_delta_rule_66_amd import recurrent_steps
    say("decode multi dtype=%s K=%d V=%d T=%d" % (dtype, K, V, T))
    N, H = 5, 3
    d = make_decode(N, H, K, V, T, dtype, seed=23)
    tok = lambda t: t.transpose(0, 1).contiguous()          # [T, N, ...] -> [N, T, ...]
    xm = {n: tok(d[n]).to(DEV) for n in ("q", "k", "v", "g", "beta")}
    state = d["state"].to(DEV).clone()
    o, steps = recurrent_steps(xm["q"], xm["k"], xm["v"], xm["g"], xm["beta"], state, step_states=True)
    torch.cuda.synchronize()
    # oracle: the T tokens as a prefill of B = N sequences from the given state
    qo, ko, vo, go, bo = (tok(d[n]) for n in ("q", "k", "v", "g", "beta"))
    o_ref, s_ref = oracle.oracle_fwd(qo, ko, vo, go, bo, d["state"])
    assert o_err(o, o_ref) < TOL[dtype]
    assert s_err(state, s_ref) < TOL[dtype]
    for t in range(T):
        _, st_ref = oracle.oracle_fwd(qo[:, :t + 1], ko[:, :t + 1], vo[:, :t + 1], go[:, :t + 1], bo[:, :t + 1],
                                      d["state"])
        assert s_err(steps[:, t], st_ref) < TOL[dtype], t
    # the same tokens one decode step at a time
    x = to_dev(d)
    st1 = x["state"].clone()
    for t in range(T):
        o1 = recurrent_step(x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t], st1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o[:, t]), t
        assert torch.equal(st1, steps[:, t]), t
    assert torch.equal(st1, state)
    # without step states only o and the state are written
    state2 = d["state"].to(DEV).clone()
    o2 = recurrent_steps(xm["q"], xm["k"], xm["v"], xm["g"], xm["beta"], state2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(state2, state)


def max_rel(o, o_ref):
    # decode output [N, H, V]: chains (n, h)
    from tests.parity import max_rel_l2
    return max_rel_l2(o, o_ref, (0, 1))


# ------------------------------------------------------------------ full-size workloads
def _sampled_oracle(x, chains):
    """Oracle on selected (b, h) chains of device inputs; returns a list of
    (o_ref [1, T, 1, V], s_ref [1, 1, K, V]) in the order of `chains`.  The
    chains of one batch row go to the oracle in one call (its threads run
    over every (head, 16-column) chain of the call)."""
    by_row = {}
    for b, h in chains:
        by_row.setdefault(b, []).append(h)
    refs = {}
    for b, hs in by_row.items():
        idx = torch.tensor(hs, device=x["q"].device)
        sl = lambda t: t[b:b + 1].index_select(2, idx).contiguous().cpu()
        s0 = None if x["s0"] is None else x["s0"][b:b + 1].index_select(1, idx).cpu()
        o_ref, s_ref = oracle.oracle_fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), s0)
        for i, h in enumerate(hs):
            refs[(b, h)] = (o_ref[:, :, i:i + 1], s_ref[:, i:i + 1])
    return [refs[c] for c in chains]


@pytest.mark.parametrize("name,chains,split", [("prefill_8k", [(0, 0), (0, 7), (0, 19), (0, 31)], 0),
                                               ("prefill_8k", [(0, 3), (0, 30)], 1),
                                               ("prefill_8k", [(0, 5), (0, 26)], 2),
                                               ("prefill_32k_x8", [(0, 3), (5, 17), (7, 31), (2, 9)], 0),
                                               ("prefill_1m", [(0, 0), (0, 5), (0, 11), (0, 15)], 0)])
def test_full_size_prefill_sampled(name, chains, split):
    """Full-size workloads in the launch configuration bench.py times (the
    library's plan), checked against the oracle on sampled (b, h) chains."""
    cfg = CONFIGS[name]
    plan = (0, 0, split)
    say("full %s B=%d T=%d H=%d plan=%s, oracle on chains %s" %
        (name, cfg.B, cfg.T, cfg.H, chunk_plan(cfg.B, cfg.T, cfg.H, cfg.K, cfg.V, cfg.dtype) if not split
         else plan, chains))
    x = make_prefill_config(cfg, DEV)
    if cfg.pinned_frac:
        # the sampled heads carry gates pinned at the clamp floor
        for _, h in chains:
            assert bool(x["pinned"][h].any()), h
    o, sT = chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], True, plan)
    torch.cuda.synchronize()
    assert torch.isfinite(sT).all()
    refs = _sampled_oracle(x, chains)
    for (b, h), (o_ref, s_ref) in zip(chains, refs):
        assert o_err(o[b:b + 1, :, h:h + 1], o_ref) < TOL[cfg.dtype], (b, h)
        assert s_err(sT[b:b + 1, h:h + 1], s_ref) < TOL[cfg.dtype], (b, h)
    del x, o, sT
    torch.cuda.empty_cache()


def test_full_size_decode_sampled():
    cfg = CONFIGS["decode_256x32"]
    say("full decode workload N=%d H=%d steps=%d, oracle on 8 sequences" % (cfg.N, cfg.H, cfg.steps))
    x = make_decode_config(cfg, DEV)
    sel = torch.arange(0, cfg.N, cfg.N // 8)
    ref_state = x["state"][sel].double().cpu().numpy().copy()
    state = x["state"].clone()
    for t in range(cfg.steps):
        o = recurrent_step(x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t], state)
        o_ref = oracle.oracle_step(x["q"][t][sel].cpu(), x["k"][t][sel].cpu(), x["v"][t][sel].cpu(),
                                   x["g"][t][sel].cpu(), x["beta"][t][sel].cpu(), ref_state)
        assert max_rel(o[sel], o_ref) < TOL[cfg.dtype], t
    torch.cuda.synchronize()
    assert s_err(state[sel], ref_state) < TOL[cfg.dtype]
