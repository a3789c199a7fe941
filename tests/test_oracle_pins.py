"""Pins for the fp64 oracle: what the pages and the mathematics fix.

Each test is chosen so that a plausible mistake in the oracle (a dropped
decay, decay after instead of before the erase, read-out before the update, a
wrong sign, a transposed state, a missing clamp side) fails at least one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.kda_bruteforce import exact_chain, dense_f64_chain, segment_transition_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, K, V, unit_k=True, g_lo=-5.0):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = rng.random((B, T, H))
    g = rng.uniform(g_lo, 0.0, (B, T, H, K))
    f = lambda x: x.astype(np.float32)
    return f(q), f(k), f(v), f(g), f(beta)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 1e-30 else 1.0)


def _frac(s):
    return Fraction(s)


@pytest.mark.parametrize("name", ["kda_hand_t2.json"])
def test_golden_hand_worked_example(name):
    d = json.load(open(os.path.join(GOLDEN, name)))
    inp = d["inputs"]
    T, K = len(inp["k"]), len(inp["k"][0])
    V = len(inp["v"][0])
    arr = lambda x, sh: np.array([float(_frac(str(e))) if isinstance(e, str) else float(e)
                                  for e in np.array(x, dtype=object).ravel()]).reshape(sh)
    q = arr(inp["q"], (1, T, 1, K)).astype(np.float32)
    k = arr(inp["k"], (1, T, 1, K)).astype(np.float32)
    v = arr(inp["v"], (1, T, 1, V)).astype(np.float32)
    g = arr(inp["g"], (1, T, 1, K)).astype(np.float32)
    beta = arr(inp["beta"], (1, T, 1)).astype(np.float32)
    s0 = arr(inp["s0"], (1, 1, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    o_exp = arr(d["expected"]["o"], (T, V))
    s_exp = arr(d["expected"]["sT"], (K, V))
    np.testing.assert_allclose(o[0, :, 0, :], o_exp, rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(sT[0, 0], s_exp, rtol=1e-7, atol=1e-7)


def test_golden_clamp_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "kda_hand_clamp.json")))
    inp = d["inputs"]
    E = math.exp(-5.0)
    val = lambda e: E if e == "E" else float(Fraction(e))
    arr = lambda x, sh: np.array([val(e) if isinstance(e, str) else float(e)
                                  for e in np.array(x, dtype=object).ravel()]).reshape(sh)
    T, K, V = 2, 2, 2
    q = arr(inp["q"], (1, T, 1, K)).astype(np.float32)
    k = arr(inp["k"], (1, T, 1, K)).astype(np.float32)
    v = arr(inp["v"], (1, T, 1, V)).astype(np.float32)
    g = arr(inp["g"], (1, T, 1, K)).astype(np.float32)
    beta = arr(inp["beta"], (1, T, 1)).astype(np.float32)
    s0 = arr(inp["s0"], (1, 1, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o[0, :, 0, :], arr(d["expected"]["o"], (T, V)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sT[0, 0], arr(d["expected"]["sT"], (K, V)), rtol=1e-14, atol=1e-15)


def test_p1_no_forget_no_write_keeps_state():
    """alpha = 1, beta = 0: S_T = S0 exactly and o_t = S0^T q_t."""
    rng = np.random.default_rng(1)
    B, T, H, K, V = 2, 37, 3, 16, 24
    q, k, v, g, beta = _rand_inputs(rng, B, T, H, K, V)
    g[:] = 0.0
    beta[:] = 0.0
    s0 = rng.standard_normal((B, H, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    assert np.array_equal(sT, s0)
    ref = np.einsum("bhkv,bthk->bthv", s0, q.astype(np.float64))
    assert _rel(o, ref) < 1e-13


def test_p2_full_write_unit_key_reproduces_value():
    """alpha = 1, beta = 1, ||k|| = 1: S_t^T k_t = v_t, so q_t = k_t gives o_t = v_t."""
    rng = np.random.default_rng(2)
    B, T, H, K, V = 1, 50, 2, 8, 5
    # basis keys: exactly unit in any precision
    idx = rng.integers(0, K, size=(B, T, H))
    k = np.zeros((B, T, H, K), np.float32)
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    q = k.copy()
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    g = np.zeros((B, T, H, K), np.float32)
    beta = np.ones((B, T, H), np.float32)
    s0 = rng.standard_normal((B, H, K, V))
    o, _ = oracle.oracle_fwd(q, k, v, g, beta, s0)
    np.testing.assert_allclose(o, v.astype(np.float64), rtol=0, atol=1e-12)
    # general unit keys (unit up to fp32 rounding of the normalised vector)
    q2, k2, v2, _, _ = _rand_inputs(rng, B, T, H, K, V)
    o2, _ = oracle.oracle_fwd(k2, k2, v2, g, beta, s0)
    np.testing.assert_allclose(o2, v2.astype(np.float64), rtol=0, atol=1e-5)


def test_p3_clamp_both_sides_bitwise():
    rng = np.random.default_rng(3)
    B, T, H, K, V = 1, 40, 2, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    lo = np.full_like(g, -5.0)
    lo2 = np.full_like(g, -50.0)
    hi = np.zeros_like(g)
    hi2 = np.full_like(g, 3.0)
    a = oracle.oracle_fwd(q, k, v, lo, beta, s0)
    b = oracle.oracle_fwd(q, k, v, lo2, beta, s0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    a = oracle.oracle_fwd(q, k, v, hi, beta, s0)
    b = oracle.oracle_fwd(q, k, v, hi2, beta, s0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # mixed: out-of-range channels clamp independently
    gm = g.copy()
    gm[..., ::2] = -9.0
    gm[..., 1::4] = 0.7
    gc = gm.copy()
    gc[..., ::2] = -5.0
    gc[..., 1::4] = 0.0
    a = oracle.oracle_fwd(q, k, v, gm, beta, s0)
    b = oracle.oracle_fwd(q, k, v, gc, beta, s0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_p4_pure_decay_closed_form():
    """beta = 0: S_T = Diag(exp(sum_t clamp g_t)) S0, o_t = (Diag(e^{G_t}) S0)^T q_t."""
    rng = np.random.default_rng(4)
    B, T, H, K, V = 2, 30, 2, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, B, T, H, K, V, g_lo=-1.0)
    g[..., 0] = -7.0   # below the floor: acts as -5
    g[..., 1] = 0.5    # above the ceiling: acts as 0
    beta[:] = 0.0
    s0 = rng.standard_normal((B, H, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    G = np.cumsum(np.clip(g.astype(np.float64), -5.0, 0.0), axis=1)  # [B,T,H,K]
    s_ref = np.exp(G[:, -1])[..., None] * s0
    assert _rel(sT, s_ref) < 1e-12
    o_ref = np.einsum("bthk,bhkv,bthk->bthv", np.exp(G), s0, q.astype(np.float64))
    assert _rel(o, o_ref) < 1e-12


@pytest.mark.parametrize("T,K,V,seed", [(1, 3, 2, 10), (3, 4, 3, 11), (6, 5, 4, 12), (8, 3, 5, 13)])
def test_p5_exact_rational_brute_force(T, K, V, seed):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, K, V, unit_k=False)
    g[0, :, 0, 0] = -6.0  # one channel beyond the floor
    s0 = rng.standard_normal((1, 1, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    oe, se = exact_chain(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], s0[0, 0])
    oe = np.array([[float(x) for x in r] for r in oe])
    se = np.array([[float(x) for x in r] for r in se])
    assert _rel(o[0, :, 0], oe) < 1e-13
    assert _rel(sT[0, 0], se) < 1e-13


def test_p5_dense_expansion_wider():
    rng = np.random.default_rng(14)
    T, K, V = 7, 32, 16
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, K, V)
    s0 = rng.standard_normal((1, 1, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    od, sd = dense_f64_chain(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], s0[0, 0])
    assert _rel(o[0, :, 0], od) < 1e-12
    assert _rel(sT[0, 0], sd) < 1e-12


def test_p6_segment_recombination_exact():
    """S_T = P2 (P1 S0 + L1) + L2 for a split at any point (fp64)."""
    rng = np.random.default_rng(6)
    T, K, V = 29, 12, 7
    q, k, v, g, beta = _rand_inputs(rng, 1, T, 1, K, V)
    s0 = rng.standard_normal((1, 1, K, V))
    _, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    for cut in (1, 11, 28):
        sl1, sl2 = slice(0, cut), slice(cut, T)
        P1 = segment_transition_f64(k[0, sl1, 0], g[0, sl1, 0], beta[0, sl1, 0])
        P2 = segment_transition_f64(k[0, sl2, 0], g[0, sl2, 0], beta[0, sl2, 0])
        _, L1 = oracle.oracle_fwd(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1], None)
        _, L2 = oracle.oracle_fwd(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], beta[:, sl2], None)
        comb = P2 @ (P1 @ s0[0, 0] + L1[0, 0]) + L2[0, 0]
        assert _rel(comb, sT[0, 0]) < 1e-12
        # split and resume from the fp64 mid state
        o1, s1 = oracle.oracle_fwd(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1], s0)
        o2, s2 = oracle.oracle_fwd(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], beta[:, sl2], s1)
        assert np.array_equal(s2, sT)


def test_p7_linear_in_state_and_values():
    rng = np.random.default_rng(7)
    B, T, H, K, V = 1, 45, 2, 10, 9
    q, k, v, g, beta = _rand_inputs(rng, B, T, H, K, V)
    s0 = rng.standard_normal((B, H, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    oa, sa = oracle.oracle_fwd(q, k, np.zeros_like(v), g, beta, s0)
    ob, sb = oracle.oracle_fwd(q, k, v, g, beta, None)
    assert _rel(oa + ob, o) < 1e-12
    assert _rel(sa + sb, sT) < 1e-12


def test_decode_step_matches_one_token_forward():
    rng = np.random.default_rng(8)
    N, H, K, V = 3, 2, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, N, 1, H, K, V)
    s0 = rng.standard_normal((N, H, K, V))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    st = s0.copy()
    o1 = oracle.oracle_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], st)
    assert np.array_equal(o1, o[:, 0])
    assert np.array_equal(st, sT)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(9)
    q, k, v, g, beta = _rand_inputs(rng, 2, 0, 2, 4, 4)
    s0 = rng.standard_normal((2, 2, 4, 4))
    o, sT = oracle.oracle_fwd(q, k, v, g, beta, s0)
    assert o.shape == (2, 0, 2, 4)
    assert np.array_equal(sT, s0)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(10)
    q, k, v, g, beta = _rand_inputs(rng, 2, 33, 3, 16, 40)
    a = oracle.oracle_fwd(q, k, v, g, beta, None, nthreads=1)
    b = oracle.oracle_fwd(q, k, v, g, beta, None, nthreads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
