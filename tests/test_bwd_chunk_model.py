"""The chunk form of the backward, modelled in numpy, against the fp64 oracle.

The GPU backward differentiates the chunk form of the forward (per 16-token
chunk with entering state S0: K+ = K e^G, K- = K e^-G, Q+ = Q e^G,
Ke = K e^(G_last - G), gam = e^G_last, A = StrictTril(diag(b) K+ K-^T),
M = Tril(Q+ K-^T), T = (I + A)^-1, Delta = T diag(b) (V - K+ S0)).  This file
writes those formulas once more in numpy (a model of the algorithm the kernels
implement, not of their code) and checks, on one chunk with strong and weak
gates:

* every gradient of the model equals the oracle's token-by-token derivative
  (oracle.kda_backward) to fp64 rounding;
* dlog_alpha written as the sum over the gate pairs each alpha_t enters equals
  the suffix sum of dG in fp64, and evaluated in fp32 keeps its relative
  precision at a -30 gate where the suffix-sum form loses every digit (the
  reason the gradient kernel sums the pairs).
"""
import numpy as np

import oracle

C, D = 16, 8


def _case(seed=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((C, D))
    k = rng.standard_normal((C, D)) / np.sqrt(D)
    v = rng.standard_normal((C, D))
    b = rng.uniform(0.1, 0.9, C)
    g = -np.abs(rng.standard_normal((C, D))) * 0.5
    g[5, 2] = -30.0  # alpha ~ 1e-13 in one channel of one token
    g[9, :3] = -12.0
    S0 = rng.standard_normal((D, D)) * 0.3   # [k][v]
    dO = rng.standard_normal((C, D))
    dSC = rng.standard_normal((D, D)) * 0.2  # dL/dS at the chunk end, [k][v]
    return q, k, v, b, g, S0, dO, dSC


def _model(q, k, v, b, g, S0, dO, dSC, dt):
    """Forward and backward of one chunk in the chunk form, all in dtype dt."""
    q, k, v, b, g, S0, dO, dSC = (np.asarray(x, dt) for x in (q, k, v, b, g, S0, dO, dSC))
    G = np.cumsum(g, axis=0)
    Kp, Km, Qp = k * np.exp(G), k * np.exp(-G), q * np.exp(G)
    Ke, gam = k * np.exp(G[-1] - G), np.exp(G[-1])
    A = np.tril(b[:, None] * (Kp @ Km.T), -1)
    M = np.tril(Qp @ Km.T)
    T = np.linalg.inv(np.eye(C, dtype=dt) + A).astype(dt)
    X = v - Kp @ S0
    Dl = T @ (b[:, None] * X)
    O = Qp @ S0 + M @ Dl
    SC = gam[:, None] * S0 + Ke.T @ Dl
    # backward
    dDl = M.T @ dO + Ke @ dSC
    lam = T.T @ dDl
    dX = b[:, None] * lam
    dA = -np.tril(lam @ Dl.T, -1)
    P = b[:, None] * dA
    dM = np.tril(dO @ Dl.T)
    dqs, xs, dke = dO @ S0.T, dX @ S0.T, Dl @ dSC.T
    s1 = np.sum(S0 * dSC, axis=1)
    dQp = dqs + dM @ Km
    dKp = -xs + P @ Km
    dKm = dM.T @ Qp + P.T @ Kp
    grads = {
        "dq": dQp * np.exp(G),
        "dk": dKp * np.exp(G) + dKm * np.exp(-G) + dke * np.exp(G[-1] - G),
        "dv": dX,
        "dbeta": np.sum(X * lam, axis=1) + np.sum(dA * (Kp @ Km.T), axis=1),
        "dstate0": (gam[:, None] * dSC + Qp.T @ dO - Kp.T @ dX).T,  # stored [v][k]
    }
    # dlog_alpha, suffix-sum form
    dG = dQp * Qp + dKp * Kp - dKm * Km - dke * Ke
    dG[-1] += gam * s1 + np.sum(dke * Ke, axis=0)
    suffix = np.cumsum(dG[::-1], axis=0)[::-1]
    # dlog_alpha, sum over the gate pairs each alpha_t enters
    pairs = np.zeros((C, D), dt)
    u = dqs * Qp - xs * Kp
    w = dke * Ke
    for t in range(C):
        pairs[t] = u[t:].sum(0) + w[:t].sum(0) + gam * s1
        for i in range(t, C):
            for j in range(t):
                pairs[t] += (dM[i, j] * Qp[i] + P[i, j] * Kp[i]) * Km[j]
    return O, SC, grads, suffix, pairs


def _oracle(q, k, v, b, g, S0, dO, dSC):
    f = lambda x: np.ascontiguousarray(x[:, None])
    st = np.array([0, C])
    out, fin = oracle.kda_forward(f(q), f(k), f(v), f(g), b[:, None],
                                  state0=S0.T[None, None].copy(), seq_start=st)
    res = oracle.kda_backward(f(q), f(k), f(v), f(g), b[:, None], f(dO),
                              d_state=dSC.T[None, None].copy(), state0=S0.T[None, None].copy(),
                              seq_start=st)
    return out[:, 0], fin[0, 0], res


def test_chunk_form_gradients_equal_the_oracle():
    case = _case()
    O, SC, grads, suffix, pairs = _model(*case, np.float64)
    out, fin, ref = _oracle(*case)
    assert np.abs(O - out).max() < 1e-12
    assert np.abs(SC.T - fin).max() < 1e-12
    for name in ("dq", "dk", "dv", "dbeta"):
        assert np.abs(grads[name] - ref[name][:, 0]).max() < 1e-11, name
    assert np.abs(grads["dstate0"] - ref["dstate0"][0, 0]).max() < 1e-11
    scale = np.abs(ref["dlog_alpha"]).max()
    assert np.abs(suffix - ref["dlog_alpha"][:, 0]).max() < 1e-11 * scale
    assert np.abs(pairs - ref["dlog_alpha"][:, 0]).max() < 1e-11 * scale


def test_pair_sum_keeps_precision_where_suffix_sum_cancels():
    case = _case()
    _, _, ref = _oracle(*case)
    exact = ref["dlog_alpha"][:, 0]
    _, _, _, suffix, pairs = _model(*case, np.float32)
    rel = lambda x: np.abs(x - exact) / np.abs(exact)
    # the -30 gate's entry: ~1e-14 in size, the terms of the suffix sum O(1)
    assert abs(exact[5, 2]) < 1e-10
    assert rel(pairs).max() < 1e-4
    assert rel(suffix)[5, 2] > 1.0
