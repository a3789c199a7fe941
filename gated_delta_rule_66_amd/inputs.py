"""Seeded synthetic inputs for KDA prefill and decode.

This module holds only the input recipe (distributions, shapes, seeds); none
of the method's arithmetic.  Both the HIP path and the fp64 oracle are fed
from it.  All draws are fp32 normals from one seeded ``torch.Generator`` in a
fixed order (q, k, v, beta-noise, g-noise, initial state, channel mask), then
shaped and cast:

* q, k : N(0, 1) rows, L2-normalised over the key dimension per (b, t, h);
* v    : N(0, 1);
* beta : sigmoid(N(0, 1))                       -- write strength in (0, 1);
* g    : clamp(-softplus(N(0, 1) + 2), -5, 0)   -- log forget gate;
* s0   : N(0, 1) * s0_std (fp32) when requested;
* pinned channels: a seeded set of floor(frac * H * K) (head, channel) pairs,
  shared by every batch row and token, whose g is exactly -5 (the floor of
  the forget-gate clamp).

Casting to bf16 (round to nearest even) happens after normalisation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    dtype: torch.dtype
    seed: int
    s0_std: Optional[float] = None      # None: zero initial state
    pinned_frac: float = 0.0            # share of (h, c) pairs with g = -5
    want_final: bool = True


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    K: int
    V: int
    steps: int
    dtype: torch.dtype
    seed: int
    s_std: float = 0.02


# The five workloads: a small fp32 correctness case, a single 8K sequence,
# a batch of 32K sequences from a random state with 20% of channels at the
# gate floor, one 1M-token sequence on 16 heads, and 64 decode steps over
# 256 sequences with a 512 MiB fp32 state.
CONFIGS = {
    "prefill_small_fp32": PrefillConfig("prefill_small_fp32", B=1, T=256, H=2, K=64, V=64, dtype=torch.float32, seed=0),
    "prefill_8k": PrefillConfig("prefill_8k", B=1, T=8192, H=32, K=128, V=128, dtype=torch.bfloat16, seed=1),
    "prefill_32k_x8": PrefillConfig("prefill_32k_x8", B=8, T=32768, H=32, K=128, V=128, dtype=torch.bfloat16, seed=2,
                        s0_std=0.02, pinned_frac=0.2),
    "prefill_1m": PrefillConfig("prefill_1m", B=1, T=1048576, H=16, K=128, V=128, dtype=torch.bfloat16, seed=3),
    "decode_256x32": DecodeConfig("decode_256x32", N=256, H=32, K=128, V=128, steps=64, dtype=torch.bfloat16, seed=4),
}


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _l2norm_rows(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-12)


def make_prefill(B, T, H, K, V, dtype=torch.bfloat16, seed=0, device="cpu",
                 s0_std=None, pinned_frac=0.0):
    """Inputs for one prefill call; returns a dict of tensors on ``device``.

    Keys: q, k, g [B,T,H,K]; v [B,T,H,V]; beta [B,T,H] (all ``dtype``);
    s0 [B,H,K,V] fp32 or None; pinned: bool [H,K] mask of g = -5 channels.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    q = _l2norm_rows(_normal((B, T, H, K), gen, dev)).to(dtype)
    k = _l2norm_rows(_normal((B, T, H, K), gen, dev)).to(dtype)
    v = _normal((B, T, H, V), gen, dev).to(dtype)
    beta = torch.sigmoid(_normal((B, T, H), gen, dev)).to(dtype)
    g = (-torch.nn.functional.softplus(_normal((B, T, H, K), gen, dev) + 2.0)).clamp_(-5.0, 0.0)
    s0 = None
    if s0_std is not None:
        s0 = _normal((B, H, K, V), gen, dev) * float(s0_std)
    pinned = torch.zeros((H, K), dtype=torch.bool, device=dev)
    n_pin = int(math.floor(pinned_frac * H * K))
    if n_pin > 0:
        idx = torch.randperm(H * K, generator=gen, device=dev)[:n_pin]
        pinned.view(-1)[idx] = True
        g = torch.where(pinned.view(1, 1, H, K), torch.full_like(g, -5.0), g)
    g = g.to(dtype)
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0, pinned=pinned)


def make_prefill_config(cfg: PrefillConfig, device="cpu", T=None, B=None, H=None):
    """Inputs for a named prefill workload (optionally with fewer B/T/H)."""
    return make_prefill(B if B is not None else cfg.B, T if T is not None else cfg.T,
                        H if H is not None else cfg.H, cfg.K, cfg.V, cfg.dtype, cfg.seed,
                        device, cfg.s0_std, cfg.pinned_frac)


def make_decode(N, H, K, V, steps, dtype=torch.bfloat16, seed=4, device="cpu", s_std=0.02):
    """Inputs for ``steps`` successive decode steps, drawn up front.

    Keys: q, k, g [steps,N,H,K]; v [steps,N,H,V]; beta [steps,N,H] (``dtype``);
    state [N,H,K,V] fp32 with N(0,1)*s_std entries.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    q = _l2norm_rows(_normal((steps, N, H, K), gen, dev)).to(dtype)
    k = _l2norm_rows(_normal((steps, N, H, K), gen, dev)).to(dtype)
    v = _normal((steps, N, H, V), gen, dev).to(dtype)
    beta = torch.sigmoid(_normal((steps, N, H), gen, dev)).to(dtype)
    g = (-torch.nn.functional.softplus(_normal((steps, N, H, K), gen, dev) + 2.0)).clamp_(-5.0, 0.0).to(dtype)
    state = _normal((N, H, K, V), gen, dev) * float(s_std)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state=state)


def make_decode_config(cfg: DecodeConfig, device="cpu", N=None, steps=None):
    return make_decode(N if N is not None else cfg.N, cfg.H, cfg.K, cfg.V,
                       steps if steps is not None else cfg.steps, cfg.dtype, cfg.seed,
                       device, cfg.s_std)
