"""Exact-rational brute force of the KDA recurrence (second oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). It is written in a
different form from the C oracle: the per-token transition matrix
  S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
  o_t = S_t^T q_t,
which expands the decay-then-correct update of
  "Kimi K3 发布核实与 Moonshot AI 主干架构演变", section 3, paragraph
  "KDA 为什么不同于 MLA" (decay by alpha_t, correct with beta_t, k_t, v_t,
  read the query from the updated state)
and the delta rule of
  "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE", section 二.3
  (write back only the difference between v_t and what the key reads).
Expanding: D S - beta k k^T D S + beta k v^T = D S + beta k (v - (D S)^T k)^T.
Works over any number type; with ``fractions.Fraction`` it is exact.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def transition_form(q, k, v, alpha, beta, S0):
    """One head. q, k, alpha: T rows of length K; v: T rows of length V;
    beta: T scalars; S0: K x V. Returns (o: T rows of length V, S_T)."""
    K = len(k[0])
    V = len(v[0])
    S = [list(row) for row in S0]
    outs = []
    for t in range(len(k)):
        kt, vt, at, bt, qt = k[t], v[t], alpha[t], beta[t], q[t]
        M = [[(1 if i == j else 0) - bt * kt[i] * kt[j] for j in range(K)] for i in range(K)]
        DS = [[at[i] * S[i][c] for c in range(V)] for i in range(K)]
        S = [[sum(M[i][j] * DS[j][c] for j in range(K)) + bt * kt[i] * vt[c] for c in range(V)]
             for i in range(K)]
        outs.append([sum(S[i][c] * qt[i] for i in range(K)) for c in range(V)])
    return outs, S


def rational_problem(seed, T, K, V):
    """Tiny exact problem: alpha in (0, 1], beta in [0, 1], small rationals elsewhere."""
    r = np.random.default_rng(seed)

    def fr(lo, hi, den):
        return Fraction(int(r.integers(lo * den, hi * den + 1)), den)

    alpha = [[fr(0, 1, 8) or Fraction(1, 16) for _ in range(K)] for _ in range(T)]
    beta = [fr(0, 1, 4) for _ in range(T)]
    k = [[fr(-2, 2, 3) for _ in range(K)] for _ in range(T)]
    q = [[fr(-2, 2, 5) for _ in range(K)] for _ in range(T)]
    v = [[fr(-3, 3, 2) for _ in range(V)] for _ in range(T)]
    S0 = [[fr(-1, 1, 7) for _ in range(V)] for _ in range(K)]
    return q, k, v, alpha, beta, S0
