"""Pins of the fp64 backward oracle (``oracle.kda_backward``).

The pages give the forward recurrence only, so the backward oracle is pinned
against the forward oracle itself through finite differences (an independent
route to the same derivatives), against closed forms of a special case that
reduce the recurrence to a constant state, and against its own split/resume
consistency across the checkpoint blocks it recomputes from.

Loss used throughout: L = sum(d_out * out) + sum(d_state * final_state), so
the gradients the backward returns for (d_out, d_state) are dL/d(input).
"""
import numpy as np
import pytest

import oracle


def case(lens, H, dk, dv, seed, beta_zero=False, alpha_one=False):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -np.log1p(np.exp(rng.standard_normal((T, H, dk)) - 1.0))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    if beta_zero:
        b[:] = 0.0
    if alpha_one:
        la[:] = 0.0
    N = len(lens)
    s0 = 0.3 * rng.standard_normal((N, H, dv, dk))
    do = rng.standard_normal((T, H, dv))
    ds = rng.standard_normal((N, H, dv, dk))
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b, state0=s0, d_out=do, d_state=ds,
                seq_start=starts)


NAMES = ("q", "k", "v", "log_alpha", "beta", "state0")
GRAD = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "beta": "dbeta",
        "state0": "dstate0"}


def loss(c, **over):
    x = {n: over.get(n, c[n]) for n in NAMES}
    out, fin = oracle.kda_forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                                  state0=x["state0"], seq_start=c["seq_start"])
    return float(np.sum(c["d_out"] * out) + np.sum(c["d_state"] * fin))


def grads(c):
    return oracle.kda_backward(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["d_out"],
                               d_state=c["d_state"], state0=c["state0"],
                               seq_start=c["seq_start"])


def test_backward_matches_central_differences_element_by_element():
    """Two packed sequences (4 and 3 tokens), H=2, d_k=4, d_v=3: every input
    element perturbed on its own."""
    c = case([4, 3], H=2, dk=4, dv=3, seed=1)
    g = grads(c)
    h = 1e-6
    for name in NAMES:
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (loss(c, **{name: xp}) - loss(c, **{name: xm})) / (2 * h)
        err = np.max(np.abs(fd - g[GRAD[name]])) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("name", NAMES)
def test_backward_directional_derivative_across_checkpoint_blocks(name):
    """150 tokens (the oracle recomputes states from checkpoints every 64):
    a random direction in one input, central difference against <grad, u>."""
    c = case([150], H=1, dk=8, dv=6, seed=2)
    g = grads(c)
    rng = np.random.default_rng(3)
    u = rng.standard_normal(c[name].shape)
    h = 1e-6
    fd = (loss(c, **{name: c[name] + h * u}) - loss(c, **{name: c[name] - h * u})) / (2 * h)
    an = float(np.sum(g[GRAD[name]] * u))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_backward_constant_state_closed_form():
    """beta = 0 and alpha = 1 freeze the state at S_0, so o_t = S_0^T q_t and
    every gradient has a closed form (written here with S = M^T directly)."""
    c = case([5, 9], H=2, dk=4, dv=3, seed=4, beta_zero=True, alpha_one=True)
    g = grads(c)
    st = c["seq_start"]
    for n in range(2):
        for h in range(2):
            S0 = c["state0"][n, h].T                      # [d_k, d_v]
            G = c["d_state"][n, h].T.copy()
            for t in range(st[n + 1] - 1, st[n] - 1, -1):
                qt, kt, vt, dot = c["q"][t, h], c["k"][t, h], c["v"][t, h], c["d_out"][t, h]
                G = G + np.outer(qt, dot)                 # dL/dS_t
                assert np.allclose(g["dq"][t, h], S0 @ dot, atol=1e-12)
                assert np.allclose(g["dv"][t, h], 0.0, atol=1e-12)
                assert np.allclose(g["dk"][t, h], 0.0, atol=1e-12)
                # beta enters as beta k (v - S0^T k)^T
                assert np.isclose(g["dbeta"][t, h], (G.T @ kt) @ (vt - S0.T @ kt), atol=1e-12)
                # log_alpha enters as Diag(exp(log_alpha)) S_prev at log_alpha = 0
                assert np.allclose(g["dlog_alpha"][t, h], np.sum(G * S0, axis=1), atol=1e-12)
            assert np.allclose(g["dstate0"][n, h], G.T, atol=1e-12)


def test_backward_split_resume():
    """The backward of a sequence equals the backward of its second part
    followed by that of its first part, seeded with the second part's initial
    state gradient (split at token 100, away from the 64-token checkpoints)."""
    c = case([230], H=2, dk=6, dv=5, seed=5)
    g = grads(c)
    cut = 100
    s1 = {n: c[n][:cut] for n in ("q", "k", "v", "log_alpha", "beta", "d_out")}
    s2 = {n: c[n][cut:] for n in ("q", "k", "v", "log_alpha", "beta", "d_out")}
    _, mid = oracle.kda_forward(s1["q"], s1["k"], s1["v"], s1["log_alpha"], s1["beta"],
                                state0=c["state0"])
    g2 = oracle.kda_backward(s2["q"], s2["k"], s2["v"], s2["log_alpha"], s2["beta"],
                             s2["d_out"], d_state=c["d_state"], state0=mid)
    g1 = oracle.kda_backward(s1["q"], s1["k"], s1["v"], s1["log_alpha"], s1["beta"],
                             s1["d_out"], d_state=g2["dstate0"], state0=c["state0"])
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        assert np.allclose(np.concatenate([g1[key], g2[key]]), g[key], rtol=1e-10, atol=1e-12)
    assert np.allclose(g1["dstate0"], g["dstate0"], rtol=1e-10, atol=1e-12)
