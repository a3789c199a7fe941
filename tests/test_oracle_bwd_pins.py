"""Pins of the oracle's backward (``oracle_bwd``) against things other than
its own formulas: central finite differences of the oracle's forward, an
independent fp64 autograd of the recurrence, the clamp's zero gradient, and
linearity in the incoming gradients.  CPU only."""
import numpy as np
import pytest
import torch

import oracle


def _inputs(B, T, H, K, V, seed, g_lo=-4.5, g_hi=-0.2):
    rng = np.random.default_rng(seed)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    q = f32(rng.standard_normal((B, T, H, K)))
    k = rng.standard_normal((B, T, H, K))
    k = f32(k / np.linalg.norm(k, axis=-1, keepdims=True))
    v = f32(rng.standard_normal((B, T, H, V)))
    g = f32(rng.uniform(g_lo, g_hi, (B, T, H, K)))
    beta = f32(rng.uniform(0.05, 0.95, (B, T, H)))
    s0 = rng.standard_normal((B, H, K, V)) * 0.3
    d_o = f32(rng.standard_normal((B, T, H, V)))
    dsT = rng.standard_normal((B, H, K, V))
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0), d_o, dsT


def _loss(x, d_o, dsT):
    o, sT = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"])
    return float((o * d_o).sum() + (sT * dsT).sum())


@pytest.mark.parametrize("T", [5, 70])
def test_backward_matches_finite_differences(T):
    """L = <o, dO> + <S_T, dS_T>; every gradient entry sampled against
    (L(x+) - L(x-)) / (x+ - x-), with x+- the fp32 numbers the forward
    actually receives (token inputs are fp32 on the oracle's interface)."""
    x, d_o, dsT = _inputs(1, T, 2, 6, 5, seed=T)
    grads = dict(zip(("q", "k", "v", "g", "beta", "s0"),
                     oracle.oracle_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, dsT)))
    rng = np.random.default_rng(100 + T)
    for name, grad in grads.items():
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in grad.shape)
            base = x[name][idx]
            h = 1e-3 * max(1.0, abs(base))
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            if name == "s0":
                xp[name][idx] = base + h
                xm[name][idx] = base - h
            else:   # the perturbed values as fp32, as the forward reads them
                xp[name][idx] = float(np.float32(base + h))
                xm[name][idx] = float(np.float32(base - h))
            fd = (_loss(xp, d_o, dsT) - _loss(xm, d_o, dsT)) / (xp[name][idx] - xm[name][idx])
            assert abs(fd - grad[idx]) <= 2e-5 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def _torch_forward(q, k, v, g, beta, s0):
    """The recurrence once more, in torch fp64 (for autograd)."""
    B, T, H, K = q.shape
    S = s0.clone()
    outs = []
    for t in range(T):
        a = torch.exp(torch.clamp(g[:, t], -5.0, 0.0))                 # [B, H, K]
        S = a[..., None] * S
        y = torch.einsum("bhkv,bhk->bhv", S, k[:, t])
        u = beta[:, t][..., None] * (v[:, t] - y)
        S = S + k[:, t][..., None] * u[:, :, None, :]
        outs.append(torch.einsum("bhkv,bhk->bhv", S, q[:, t]))
    return torch.stack(outs, 1), S


def test_backward_matches_independent_autograd():
    x, d_o, dsT = _inputs(2, 9, 2, 4, 3, seed=7, g_lo=-7.0, g_hi=1.0)   # some gates outside the clamp
    tx = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    o, sT = _torch_forward(tx["q"], tx["k"], tx["v"], tx["g"], tx["beta"], tx["s0"])
    ((o * torch.tensor(d_o)).sum() + (sT * torch.tensor(dsT)).sum()).backward()
    ours = oracle.oracle_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], d_o, dsT)
    for name, mine in zip(("q", "k", "v", "g", "beta", "s0"), ours):
        ref = tx[name].grad.numpy()
        assert np.allclose(mine, ref, rtol=1e-10, atol=1e-12), name


def test_backward_clamp_and_linearity():
    x, d_o, dsT = _inputs(1, 12, 1, 4, 4, seed=9)
    x["g"][0, 3, 0, 1] = -6.5          # below the clamp
    x["g"][0, 7, 0, 2] = 0.75          # above it
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"])
    r1 = oracle.oracle_bwd(*args, d_o, dsT)
    assert r1[3][0, 3, 0, 1] == 0.0 and r1[3][0, 7, 0, 2] == 0.0
    r2 = oracle.oracle_bwd(*args, 2.0 * d_o, 2.0 * dsT)   # doubling is exact in fp32 and fp64
    for a, b in zip(r1, r2):
        assert np.array_equal(2.0 * a, b)
    # no incoming gradient: every gradient is exactly zero
    for a in oracle.oracle_bwd(*args, None, None):
        assert not np.any(a)
