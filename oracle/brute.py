"""Exact rational evaluation of the gated delta rule for tiny cases (TEST INFRASTRUCTURE).

Independent of ``gdn_oracle.c``: instead of the per-token rank-1 update it multiplies out
the transition matrices. From the rule on page "Qwen3-Next -- How a running memory and a
searchable history cooperate", section "Correcting a memory instead of adding to it"
(decay, then a beta-strength correction along the key), each token applies the affine map

    S -> S M_t + beta_t v_t k_t^T,   M_t = alpha_t (I - beta_t k_t k_t^T),

so after T tokens

    S_T = S_0 M_1 M_2 ... M_T + sum_t beta_t v_t k_t^T M_{t+1} ... M_T,

and the read-out is o_t = scale * S_t q_t (after the update, as in the token loop of the
"01 . GatedDeltaNet(config)" section of "Qwen3-Next 80B-A3B -- The Evolving Transformer").
All arithmetic is on ``fractions.Fraction``; alpha, beta, keys and values must be given as
exact rationals. Pure Python loops: keep T <= 8 and d <= 4.
"""

from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence

Mat = List[List[Fraction]]


def _eye(n: int) -> Mat:
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _matmul(A: Mat, B: Mat) -> Mat:
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][r] * B[r][j] for r in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _add(A: Mat, B: Mat) -> Mat:
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _outer(x: Sequence[Fraction], y: Sequence[Fraction], c: Fraction) -> Mat:
    return [[c * xi * yj for yj in y] for xi in x]


def transition(alpha: Fraction, beta: Fraction, k: Sequence[Fraction]) -> Mat:
    """M = alpha * (I - beta * k k^T)."""
    d = len(k)
    I = _eye(d)
    return [[alpha * (I[i][j] - beta * k[i] * k[j]) for j in range(d)] for i in range(d)]


def unrolled_chain(S0: Mat, qs, ks, vs, alphas, betas, scale=Fraction(1)):
    """States S_1..S_T and outputs o_1..o_T of one chain from the unrolled product form.

    Each S_t is evaluated from scratch (no reuse of S_{t-1}), which is the brute force.
    """
    T = len(ks)
    d_k = len(S0[0])
    states, outs = [], []
    Ms = [transition(alphas[t], betas[t], ks[t]) for t in range(T)]
    for t_end in range(1, T + 1):
        P = _eye(d_k)
        for t in range(t_end):
            P = _matmul(P, Ms[t])
        S = _matmul(S0, P)
        for t in range(t_end):
            Q = _eye(d_k)
            for r in range(t + 1, t_end):
                Q = _matmul(Q, Ms[r])
            S = _add(S, _matmul(_outer(vs[t], ks[t], betas[t]), Q))
        states.append(S)
        qt = qs[t_end - 1]
        outs.append([scale * sum((S[i][j] * qt[j] for j in range(d_k)), Fraction(0))
                     for i in range(len(S))])
    return states, outs


def rank1_chain(S0: Mat, qs, ks, vs, alphas, betas, scale=Fraction(1)):
    """Same chain through the per-token form S <- a*S + b*(v - a*S k) k^T, exactly."""
    S = [row[:] for row in S0]
    states, outs = [], []
    for q, k, v, a, b in zip(qs, ks, vs, alphas, betas):
        u = [sum((S[i][j] * k[j] for j in range(len(k))), Fraction(0)) for i in range(len(S))]
        S = [[a * S[i][j] + b * (v[i] - a * u[i]) * k[j] for j in range(len(k))]
             for i in range(len(S))]
        states.append([row[:] for row in S])
        outs.append([scale * sum((S[i][j] * q[j] for j in range(len(q))), Fraction(0))
                     for i in range(len(S))])
    return states, outs


def unrolled_chain_channel(S0: Mat, qs, ks, vs, alpha_rows, betas, scale=Fraction(1)):
    """The per-channel form (code panel of section "01 . GatedDeltaNet(config)" of the
    Evolving Transformer page) by its unrolled product, row by row. Row i of the state
    evolves on its own: S_i -> S_i (alpha_i I - beta k k^T) + beta v_i k^T, so

        S_{i,T} = S_{i,0} N_1 ... N_T + sum_t beta_t v_{t,i} k_t^T N_{t+1} ... N_T,
        N_t = alpha_{t,i} I - beta_t k_t k_t^T.

    alpha_rows[t][i] is the decay of value channel i at token t. Each S_t is evaluated from
    scratch, the brute force; returns (states, outputs) as unrolled_chain does."""
    T = len(ks)
    d_v, d_k = len(S0), len(S0[0])
    I = _eye(d_k)

    def N(t, i):
        return [[alpha_rows[t][i] * I[a][b] - betas[t] * ks[t][a] * ks[t][b] for b in range(d_k)]
                for a in range(d_k)]

    states, outs = [], []
    for t_end in range(1, T + 1):
        S = []
        for i in range(d_v):
            row = [list(S0[i])]
            for t in range(t_end):
                row = _matmul(row, N(t, i))
            for t in range(t_end):
                term = [[betas[t] * vs[t][i] * kj for kj in ks[t]]]
                for s in range(t + 1, t_end):
                    term = _matmul(term, N(s, i))
                row = _add(row, term)
            S.append(row[0])
        states.append(S)
        qt = qs[t_end - 1]
        outs.append([scale * sum((S[i][j] * qt[j] for j in range(d_k)), Fraction(0)) for i in range(d_v)])
    return states, outs
