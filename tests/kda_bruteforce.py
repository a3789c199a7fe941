"""Brute-force KDA by explicit transition matrices (test helper).

A second, structurally different statement of the same recurrence as the
oracle: instead of decay / error / rank-1 update per token, each token is the
affine map  S -> A_t S + b_t k_t v_t^T  with the dense K x K matrix
A_t = (I - b_t k_t k_t^T) Diag(alpha_t).  The final state is expanded as

    S_T = A_T ... A_1 S_0 + sum_t A_T ... A_{t+1} b_t k_t v_t^T

and o_t = S_t^T q_t.  ``exact_*`` does this in exact rationals
(``fractions.Fraction``) with alpha_t = exp(clamp(g)) taken as the exact
rational value of its fp64 number; ``dense_f64`` does the same expansion in
numpy fp64.  Page: "Kimi K3 — открытая модель, которая обошла закрытых
лидеров рынка", section "Как хранить миллион токенов в памяти" (the delta
rule: previous state partly erased, new information written; alpha in
[e^-5, 1]).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _alpha_exact(gval: float) -> Fraction:
    gc = min(max(float(gval), -5.0), 0.0)
    return Fraction(math.exp(gc))


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _transition(k, b, alpha):
    """A_t = (I - b k k^T) Diag(alpha), exact."""
    K = len(k)
    return [[((1 if i == j else 0) - b * k[i] * k[j]) * alpha[j] for j in range(K)]
            for i in range(K)]


def exact_chain(q, k, v, g, beta, s0=None):
    """One chain in exact rationals.

    q, k, g: [T][K]; v: [T][V]; beta: [T]; s0: [K][V] or None.  Values are
    floats (taken exactly).  Returns (o [T][V], S_T [K][V]) as Fractions.
    """
    T = len(q)
    K = len(q[0]) if T else len(s0)
    V = len(v[0]) if T else len(s0[0])
    F = Fraction
    S0 = [[F(float(s0[i][j])) if s0 is not None else F(0) for j in range(V)] for i in range(K)]
    As, writes = [], []
    for t in range(T):
        kt = [F(float(x)) for x in k[t]]
        bt = F(float(beta[t]))
        al = [_alpha_exact(x) for x in g[t]]
        As.append(_transition(kt, bt, al))
        vt = [F(float(x)) for x in v[t]]
        writes.append([[bt * kt[i] * vt[j] for j in range(V)] for i in range(K)])
    o = []
    S_t = None
    for t in range(T):
        # S_t = A_t ... A_1 S0 + sum_{s<=t} A_t ... A_{s+1} w_s, built from the
        # explicit products (no reuse of S_{t-1}).
        acc = S0
        for s in range(t + 1):
            acc = _matmul(As[s], acc)
        for s in range(t + 1):
            term = writes[s]
            for r in range(s + 1, t + 1):
                term = _matmul(As[r], term)
            acc = [[acc[i][j] + term[i][j] for j in range(V)] for i in range(K)]
        S_t = acc
        qt = [F(float(x)) for x in q[t]]
        o.append([sum((S_t[i][j] * qt[i] for i in range(K)), F(0)) for j in range(V)])
    if S_t is None:
        S_t = S0
    return o, S_t


def dense_f64_chain(q, k, v, g, beta, s0=None):
    """The same explicit expansion in numpy fp64, for larger K, V (T small).

    Returns (o [T, V], S_T [K, V]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, K = q.shape
    V = v.shape[1]
    S0 = np.zeros((K, V)) if s0 is None else np.asarray(s0, np.float64)
    alpha = np.exp(np.clip(g, -5.0, 0.0))
    As = [(np.eye(K) - beta[t] * np.outer(k[t], k[t])) * alpha[t][None, :] for t in range(T)]
    W = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    o = np.zeros((T, V))
    S_t = S0
    for t in range(T):
        P = np.eye(K)
        for s in range(t + 1):
            P = As[s] @ P
        acc = P @ S0
        for s in range(t + 1):
            Ps = np.eye(K)
            for r in range(s + 1, t + 1):
                Ps = As[r] @ Ps
            acc = acc + Ps @ W[s]
        S_t = acc
        o[t] = S_t.T @ q[t]
    return o, S_t


def segment_transition_f64(k, g, beta):
    """P = A_T ... A_1 for a segment (fp64): how the segment maps any
    incoming state, the 'transition matrix' of a segment."""
    k = np.asarray(k, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, K = k.shape
    alpha = np.exp(np.clip(g, -5.0, 0.0))
    P = np.eye(K)
    for t in range(T):
        A = (np.eye(K) - beta[t] * np.outer(k[t], k[t])) * alpha[t][None, :]
        P = A @ P
    return P
