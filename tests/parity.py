"""Parity metric and tolerances shared by the GPU tests.

Metric: for every (batch, head) chain, the relative L2 error of the HIP
result against the fp64 oracle over that chain's outputs (T x V for o,
K x V for a state); the test takes the maximum over chains.  A chain whose
reference norm is below 1e-30 uses the absolute L2 error instead.

Tolerances: 1e-3 for fp32 inputs; 2e-2 for bf16 inputs with an fp32 state.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-3, torch.bfloat16: 2e-2}


def _np64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, np.float64)


def max_rel_l2(x, ref, chain_axes):
    """Max over chains of ||x - ref|| / ||ref||; chain_axes are the axes that
    index chains (the rest are reduced)."""
    x = _np64(x)
    ref = _np64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    red = tuple(a for a in range(x.ndim) if a not in chain_axes)
    num = np.sqrt(((x - ref) ** 2).sum(axis=red))
    den = np.sqrt((ref ** 2).sum(axis=red))
    rel = num / np.where(den < 1e-30, 1.0, den)
    if rel.size == 0:
        return 0.0
    assert np.all(np.isfinite(rel)), "non-finite error"
    return float(rel.max())


def o_err(o, o_ref):
    """o: [B, T, H, V] -> chains (b, h)."""
    return max_rel_l2(o, o_ref, (0, 2))


def s_err(s, s_ref):
    """state: [B, H, K, V] -> chains (b, h)."""
    return max_rel_l2(s, s_ref, (0, 1))
