"""Independent witnesses of the KDA recurrence, for pinning the C oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Pages cited (by title):
  [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer.

Both functions here take the math orientation S in R^{d_k x d_v} for states
([K3-explainer] §二.1) and return it in that orientation; callers transpose to
the stored [d_v, d_k] layout when they compare with ``kda_forward``.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def projection_forward(q, k, v, log_alpha, beta, S0=None):
    """One sequence, one head, explicit-matrix form of the printed KDA update.

    [K3-explainer] §四 prints the update as
        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    and §二.1 the read o_t = S_t^T q_t.  This builds the d_k x d_k matrices
    literally (fp64 numpy), a different order of operations from the C oracle's
    predict/correct loop.

    q, k, log_alpha: [T, d_k]; v: [T, d_v]; beta: [T]; S0: [d_k, d_v] or None.
    Returns (out [T, d_v], S_T [d_k, d_v]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(log_alpha, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    eye = np.eye(dk)
    out = np.zeros((T, dv))
    for t in range(T):
        erase = eye - b[t] * np.outer(k[t], k[t])
        S = erase @ np.diag(np.exp(g[t])) @ S + b[t] * np.outer(k[t], v[t])
        out[t] = S.T @ q[t]
    return out, S


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][r] * B[r][j] for r in range(m)), Fraction(0))
             for j in range(p)] for i in range(n)]


def _identity(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def transition_matrix(k_i, alpha_i, beta_i):
    """A_i = (I - beta_i k_i k_i^T) Diag(alpha_i), exact ([K3-explainer] §五)."""
    n = len(k_i)
    return [[((Fraction(int(r == c)) - beta_i * k_i[r] * k_i[c]) * alpha_i[c])
             for c in range(n)] for r in range(n)]


def brute_force_exact(q, k, v, alpha, beta, S0=None):
    """Exact-rational KDA through transition products, for tiny T and d.

    [K3-explainer] §五 states that information written at step j reaches step t
    through the product A_t A_{t-1} ... A_{j+1} with A_i = (I - beta_i k_i
    k_i^T) Diag(alpha_i).  Unrolling the update S_t = A_t S_{t-1} + beta_t k_t
    v_t^T ([K3-explainer] §四, §六's S_t = A_t S_{t-1} + B_t) gives

        S_t = (A_t ... A_1) S_0 + sum_{j<=t} (A_t ... A_{j+1}) beta_j k_j v_j^T,

    which is evaluated here term by term for every t, with no recurrence on S:
    each S_t is rebuilt from the inputs.  Output o_t = S_t^T q_t.

    All arguments are sequences of ``Fraction``-convertible numbers:
    q, k, alpha: [T][d_k]; v: [T][d_v]; beta: [T]; S0: [d_k][d_v] or None.
    ``alpha`` is the decay itself (not its log).
    Returns (out [T][d_v], S_T [d_k][d_v]) as nested lists of Fractions.
    """
    F = Fraction
    q = [[F(x) for x in row] for row in q]
    k = [[F(x) for x in row] for row in k]
    v = [[F(x) for x in row] for row in v]
    alpha = [[F(x) for x in row] for row in alpha]
    beta = [F(x) for x in beta]
    T, dk, dv = len(q), len(q[0]), len(v[0])
    S0 = ([[F(0)] * dv for _ in range(dk)] if S0 is None
          else [[F(x) for x in row] for row in S0])
    A = [transition_matrix(k[i], alpha[i], beta[i]) for i in range(T)]

    def chain(t, j):
        """A_t A_{t-1} ... A_{j+1} (0-based tokens: A[t] ... A[j+1]); I if j == t."""
        P = _identity(dk)
        for i in range(j + 1, t + 1):
            P = _matmul(A[i], P)
        return P

    out = []
    S_t = S0
    for t in range(T):
        S_t = _matmul(chain(t, -1), S0)
        for j in range(t + 1):
            write = [[beta[j] * k[j][r] * v[j][c] for c in range(dv)]
                     for r in range(dk)]
            term = _matmul(chain(t, j), write)
            S_t = [[S_t[r][c] + term[r][c] for c in range(dv)] for r in range(dk)]
        out.append([sum((S_t[r][c] * q[t][r] for r in range(dk)), F(0))
                    for c in range(dv)])
    return out, S_t
