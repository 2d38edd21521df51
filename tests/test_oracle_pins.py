"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Pages cited (by title):
  [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer.
  [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever".

None of these tests retypes the oracle's loop: each compares it with an
independent statement -- exact rational transition products, the explicit
projection form, closed forms of special cases, invariants of the update.
Most use d_k != d_v so that a transposed operand or state cannot hide.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import forms


def _rand_case(rng, T, H, dk, dv, unit_keys=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, H, dk)) - 1.0))  # log alpha < 0
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, b


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- I0 brute force
_DY = [Fraction(x, 4) for x in (-4, -3, -2, -1, 0, 1, 2, 3, 4)]
_ALPHA = [Fraction(1, 2), Fraction(3, 4), Fraction(7, 8), Fraction(1)]
_BETA = [Fraction(1, 4), Fraction(1, 2), Fraction(3, 4), Fraction(1)]


def _dyadic_case(seed, T, dk, dv, with_state=True):
    r = np.random.default_rng(seed)
    pick = lambda pool, shape: [[pool[i] for i in row] for row in r.integers(0, len(pool), shape)]
    q = pick(_DY, (T, dk))
    k = pick(_DY, (T, dk))
    v = pick(_DY, (T, dv))
    alpha = pick(_ALPHA, (T, dk))
    beta = [_BETA[i] for i in r.integers(0, len(_BETA), T)]
    S0 = pick(_DY, (dk, dv)) if with_state else None
    return q, k, v, alpha, beta, S0


@pytest.mark.parametrize("seed,T,dk,dv", [(0, 8, 3, 4), (1, 8, 4, 3), (2, 6, 4, 4),
                                          (3, 8, 2, 3), (4, 7, 4, 2)])
def test_brute_force_exact_transition_products(seed, T, dk, dv):
    """[K3-explainer] §五: S_t = (A_t..A_1)S_0 + sum_j (A_t..A_{j+1}) beta_j k_j v_j^T,
    evaluated exactly in rationals, equals the oracle to fp64 rounding."""
    q, k, v, alpha, beta, S0 = _dyadic_case(seed, T, dk, dv)
    out_x, S_x = forms.brute_force_exact(q, k, v, alpha, beta, S0)
    f = lambda rows: np.array([[float(x) for x in row] for row in rows])
    out, sT = oracle.kda_forward(
        f(q)[:, None], f(k)[:, None], f(v)[:, None],
        np.log(f(alpha))[:, None], np.array([float(b) for b in beta])[:, None],
        state0=f(S0).T[None, None])
    ref_out, ref_S = f(out_x), f(S_x)
    scale = max(np.abs(ref_out).max(), 1.0)
    assert np.abs(out[:, 0] - ref_out).max() <= 1e-13 * scale
    # stored state is S^T: [d_v, d_k]
    assert sT.shape == (1, 1, dv, dk)
    assert np.abs(sT[0, 0] - ref_S.T).max() <= 1e-13 * max(np.abs(ref_S).max(), 1.0)


# ---------------------------------------------------------------- projection form
@pytest.mark.parametrize("seed,T,dk,dv", [(0, 50, 5, 7), (1, 33, 8, 3), (2, 64, 16, 16)])
def test_projection_form_agrees(seed, T, dk, dv):
    """[K3-explainer] §四 explicit (I - b k k^T) Diag(alpha) S + b k v^T with d_k x d_k
    matrices agrees with the oracle's predict/correct loop ([K3-explainer] §三)."""
    rng = np.random.default_rng(seed)
    H = 2
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    out, sT = oracle.kda_forward(q, k, v, g, b, state0=S0)
    for h in range(H):
        o_p, S_p = forms.projection_forward(q[:, h], k[:, h], v[:, h], g[:, h], b[:, h],
                                            S0[0, h].T)
        assert _rel(out[:, h], o_p) < 1e-12
        assert _rel(sT[0, h], S_p.T) < 1e-12


# ---------------------------------------------------------------- I1: beta = 0
def test_beta_zero_is_pure_per_channel_decay():
    """beta = 0 removes the write, leaving S_t = Diag(exp(Gamma_t)) S_0 with
    Gamma_t the running sum of log alpha over tokens <= t ([K3-explainer] §四):
    o_t[j] = sum_i S_0[i][j] exp(Gamma_t[i]) q_t[i]."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 40, 3, 6, 5
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    b[:] = 0.0
    M0 = rng.standard_normal((1, H, dv, dk))
    out, sT = oracle.kda_forward(q, k, v, g, b, state0=M0)
    Gam = np.cumsum(g, axis=0)  # [T, H, dk]
    for h in range(H):
        exp_out = np.einsum("ji,ti,ti->tj", M0[0, h], np.exp(Gam[:, h]), q[:, h])
        assert _rel(out[:, h], exp_out) < 1e-13
        assert _rel(sT[0, h], M0[0, h] * np.exp(Gam[-1, h])[None, :]) < 1e-13


def test_beta_zero_alpha_one_freezes_state():
    """beta = 0, alpha = 1: nothing is written or forgotten; bitwise frozen state."""
    rng = np.random.default_rng(12)
    T, H, dk, dv = 17, 2, 4, 6
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    g[:] = 0.0
    b[:] = 0.0
    M0 = rng.standard_normal((1, H, dv, dk))
    out, sT = oracle.kda_forward(q, k, v, g, b, state0=M0)
    assert np.array_equal(sT, M0)
    for h in range(H):
        assert _rel(out[:, h], q[:, h] @ M0[0, h].T) < 1e-14


# ---------------------------------------------------------------- I2: exact retrieval
def test_unit_key_beta_one_retrieves_value_exactly():
    """With ||k_t|| = 1 and beta_t = 1, (I - k k^T) k = 0, so S_t^T k_t = v_t whatever
    alpha_t and S_{t-1} are ([K3-explainer] §三: the write replaces the old answer
    along k_t).  Reading with q_t = k_t must return v_t; this also fixes that the
    read uses S_t after the write ([K3-explainer] §二.1)."""
    rng = np.random.default_rng(13)
    T, H, dk, dv = 30, 2, 8, 5
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    b[:] = 1.0
    q = k.copy()
    M0 = rng.standard_normal((1, H, dv, dk))
    out, _ = oracle.kda_forward(q, k, v, g, b, state0=M0)
    assert np.abs(out - v).max() < 1e-12


def test_orthonormal_keys_reduce_to_linear_attention():
    """alpha = 1, beta = 1, S_0 = 0 and orthonormal keys: each write lands in a
    direction no earlier key touched, so the delta rule equals plain linear
    memory S_T = sum_t k_t v_t^T ([K3-explainer] §二.1) and every pair is
    retrievable: S_T^T k_i = v_i."""
    rng = np.random.default_rng(14)
    dk, dv = 7, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    T = dk
    k = Qm.T[:, None, :]  # rows orthonormal
    v = rng.standard_normal((T, 1, dv))
    q = rng.standard_normal((T, 1, dk))
    g = np.zeros((T, 1, dk))
    b = np.ones((T, 1))
    out, sT = oracle.kda_forward(q, k, v, g, b)
    S_lin = sum(np.outer(k[t, 0], v[t, 0]) for t in range(T))
    assert np.abs(sT[0, 0] - S_lin.T).max() < 1e-13
    retrieved = k[:, 0] @ sT[0, 0].T  # row i = (S^T k_i)^T
    assert np.abs(retrieved - v[:, 0]).max() < 1e-13


# ---------------------------------------------------------------- I3: one-hot keys
@pytest.mark.parametrize("alpha_one", [False, True])
def test_one_hot_keys_decayed_sum(alpha_one):
    """Distinct one-hot keys k_t = e_{c_t}, S_0 = 0: key row c_t is empty when
    token t arrives, so the whole value is written and then decays only through
    channel c_t's gates: row c_t of S_T = beta_t exp(Gamma_T[c_t] - Gamma_t[c_t]) v_t.
    With alpha = 1 this is sum_t beta_t k_t v_t^T ([K3-explainer] §二.1, §四)."""
    rng = np.random.default_rng(15)
    dk, dv, T = 9, 4, 6
    chans = rng.permutation(dk)[:T]
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, chans] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1, dk)) if alpha_one else -rng.uniform(0.0, 0.7, (T, 1, dk))
    b = rng.uniform(0.1, 1.0, (T, 1))
    _, sT = oracle.kda_forward(q, k, v, g, b)
    Gam = np.cumsum(g[:, 0], axis=0)
    S_exp = np.zeros((dk, dv))
    for t, c in enumerate(chans):
        S_exp[c] = b[t, 0] * np.exp(Gam[-1, c] - Gam[t, c]) * v[t, 0]
    assert np.abs(sT[0, 0] - S_exp.T).max() < 1e-14


# ---------------------------------------------------------------- I4: scalar gate
def test_scalar_gate_equals_gated_deltanet():
    """When alpha_t is equal across channels, Diag(alpha_t) = alpha_t I commutes
    with the erase and KDA is Gated DeltaNet, S_t = alpha_t (I - b k k^T) S + b k v^T
    ([K3-explainer] §四, the scalar-gate form printed before KDA's)."""
    rng = np.random.default_rng(16)
    T, dk, dv = 45, 6, 5
    q, k, v, g, b = _rand_case(rng, T, 1, dk, dv)
    g[:] = g[:, :, :1]  # one gate per token
    S = rng.standard_normal((dk, dv))
    out, sT = oracle.kda_forward(q, k, v, g, b, state0=S.T[None, None])
    o_ref = np.zeros((T, dv))
    for t in range(T):
        a = np.exp(g[t, 0, 0])
        kt = k[t, 0]
        S = a * (np.eye(dk) - b[t, 0] * np.outer(kt, kt)) @ S + b[t, 0] * np.outer(kt, v[t, 0])
        o_ref[t] = S.T @ q[t, 0]
    assert _rel(out[:, 0], o_ref) < 1e-12
    assert _rel(sT[0, 0], S.T) < 1e-12


# ---------------------------------------------------------------- delta semantics
def test_already_correct_memory_writes_nothing():
    """[K3-explainer] §三: if the decayed memory already predicts v_t, the error is
    zero and the step only decays: S_t = Diag(alpha_t) S_{t-1}."""
    rng = np.random.default_rng(17)
    T, dk, dv = 12, 5, 6
    q, k, v, g, b = _rand_case(rng, T, 1, dk, dv)
    M0 = rng.standard_normal((1, 1, dv, dk))
    _, M_prev = oracle.kda_forward(q[:-1], k[:-1], v[:-1], g[:-1], b[:-1], state0=M0)
    decayed = M_prev[0, 0] * np.exp(g[-1, 0])[None, :]  # [dv, dk]
    v_last = v.copy()
    v_last[-1, 0] = decayed @ k[-1, 0]  # = (Diag(alpha) S)^T k
    _, M_T = oracle.kda_forward(q[-1:], k[-1:], v_last[-1:], g[-1:], b[-1:], state0=M_prev)
    assert np.abs(M_T[0, 0] - decayed).max() < 1e-13


# ---------------------------------------------------------------- I6: linearity
def test_linear_in_initial_state_and_values():
    """For fixed q, k, alpha, beta the update is linear in (S_0, V)
    (every term of the §四 update is linear in S or in v)."""
    rng = np.random.default_rng(18)
    T, H, dk, dv = 25, 2, 6, 4
    q, k, v1, g, b = _rand_case(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, dv, dk))
    s2 = rng.standard_normal((1, H, dv, dk))
    a1, a2 = 0.7, -1.3
    o1, t1 = oracle.kda_forward(q, k, v1, g, b, state0=s1)
    o2, t2 = oracle.kda_forward(q, k, v2, g, b, state0=s2)
    o3, t3 = oracle.kda_forward(q, k, a1 * v1 + a2 * v2, g, b, state0=a1 * s1 + a2 * s2)
    assert _rel(o3, a1 * o1 + a2 * o2) < 1e-12
    assert _rel(t3, a1 * t1 + a2 * t2) < 1e-12


# ---------------------------------------------------------------- I5, I8, I9: structure
@pytest.mark.parametrize("T", [1, 10, 300])
def test_state_size_independent_of_length(T):
    """The state has a fixed shape whatever T is ([K3-memory] §2, §3)."""
    rng = np.random.default_rng(19)
    q, k, v, g, b = _rand_case(rng, T, 3, 4, 5)
    _, sT = oracle.kda_forward(q, k, v, g, b)
    assert sT.shape == (1, 3, 5, 4)


def test_split_and_resume_is_exact():
    """Running [0, t) then [t, T) from the first run's final state is the same
    computation, bit for bit ([K3-memory] §5: restartable state snapshots)."""
    rng = np.random.default_rng(20)
    T, H, dk, dv, t = 97, 2, 6, 5, 41
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    M0 = rng.standard_normal((1, H, dv, dk))
    o_full, s_full = oracle.kda_forward(q, k, v, g, b, state0=M0)
    o_a, s_a = oracle.kda_forward(q[:t], k[:t], v[:t], g[:t], b[:t], state0=M0)
    o_b, s_b = oracle.kda_forward(q[t:], k[t:], v[t:], g[t:], b[t:], state0=s_a)
    assert np.array_equal(np.concatenate([o_a, o_b]), o_full)
    assert np.array_equal(s_b, s_full)


def test_packed_sequences_equal_separate_runs():
    """Sequences packed along T never interact; an empty sequence returns its
    initial state."""
    rng = np.random.default_rng(21)
    lens = [13, 0, 40, 1, 7]
    starts = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = starts[-1], 2, 5, 4
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    M0 = rng.standard_normal((len(lens), H, dv, dk))
    out, sT = oracle.kda_forward(q, k, v, g, b, state0=M0, seq_start=starts)
    for n, (s, e) in enumerate(zip(starts[:-1], starts[1:])):
        o_n, s_n = oracle.kda_forward(q[s:e], k[s:e], v[s:e], g[s:e], b[s:e],
                                      state0=M0[n:n + 1])
        assert np.array_equal(out[s:e], o_n)
        assert np.array_equal(sT[n], s_n[0])
    assert np.array_equal(sT[1], M0[1])


def test_decode_steps_equal_prefill():
    """A decode step is one token of the recurrence: T single-token steps give the
    prefill's outputs and state exactly."""
    rng = np.random.default_rng(22)
    T, H, dk, dv = 20, 3, 4, 6
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    M = rng.standard_normal((1, H, dv, dk))
    o_full, s_full = oracle.kda_forward(q, k, v, g, b, state0=M)
    outs = []
    for t in range(T):
        o_t, M = oracle.kda_decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                        b[t:t + 1], M)
        outs.append(o_t)
    assert np.array_equal(np.concatenate(outs), o_full)
    assert np.array_equal(M, s_full)


def test_dense_front_end_matches_packed():
    rng = np.random.default_rng(23)
    B, T, H, dk, dv = 3, 11, 2, 4, 4
    q, k, v, g, b = _rand_case(rng, B * T, H, dk, dv)
    M0 = rng.standard_normal((B, H, dv, dk))
    o_p, s_p = oracle.kda_forward(q, k, v, g, b, state0=M0, seq_start=np.arange(B + 1) * T)
    o_d, s_d = oracle.kda_forward_dense(q.reshape(B, T, H, dk), k.reshape(B, T, H, dk),
                                        v.reshape(B, T, H, dv), g.reshape(B, T, H, dk),
                                        b.reshape(B, T, H), state0=M0)
    assert np.array_equal(o_d.reshape(B * T, H, dv), o_p)
    assert np.array_equal(s_d, s_p)


def test_rejects_bad_sequence_offsets():
    rng = np.random.default_rng(24)
    q, k, v, g, b = _rand_case(rng, 10, 1, 2, 2)
    with pytest.raises(ValueError):
        oracle.kda_forward(q, k, v, g, b, seq_start=[0, 6, 4, 10])
    with pytest.raises(ValueError):
        oracle.kda_forward(q, k, v, g, b, seq_start=[0, 11])


# ---------------------------------------------------------------- state snapshots
# [K3-memory] §5: the recurrent state kept every N tokens as a restartable
# checkpoint.  Definition: the state after the first j * N tokens of a sequence.
SNAP_LENS = [0, 5, 16, 33, 70, 96]


def _snap_case(seed, H=2, dk=6, dv=5):
    rng = np.random.default_rng(seed)
    T = sum(SNAP_LENS)
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((len(SNAP_LENS), H, dv, dk)) * 0.1
    starts = np.concatenate([[0], np.cumsum(SNAP_LENS)]).astype(np.int64)
    return q, k, v, beta, g, s0, starts


@pytest.mark.parametrize("every", [1, 16, 32])
def test_snapshots_are_the_prefix_states(every):
    q, k, v, beta, g, s0, starts = _snap_case(7)
    out, fin, snaps = oracle.kda_snapshots(q, k, v, g, beta, every, state0=s0, seq_start=starts)
    counts = [n // every for n in SNAP_LENS]
    assert snaps.shape[0] == sum(counts)
    i = 0
    for n, cnt in enumerate(counts):
        a = starts[n]
        for j in range(1, cnt + 1):
            sl = slice(a, a + j * every)
            _, ref = oracle.kda_forward(q[sl], k[sl], v[sl], g[sl], beta[sl], state0=s0[n:n + 1])
            assert _rel(snaps[i], ref[0]) < 1e-13
            i += 1
    # outputs and final states are those of the uninterrupted recurrence
    out_ref, fin_ref = oracle.kda_forward(q, k, v, g, beta, state0=s0, seq_start=starts)
    assert _rel(out, out_ref) < 1e-13 and _rel(fin, fin_ref) < 1e-13


def test_snapshots_beta_zero_closed_form():
    """beta = 0: snapshot j is the initial state decayed per channel over the
    first j * N tokens, M[v, c] * exp(sum of log_alpha[:, c])."""
    q, k, v, beta, g, s0, starts = _snap_case(8)
    every = 16
    _, _, snaps = oracle.kda_snapshots(q, k, v, g, np.zeros_like(beta), every, state0=s0,
                                       seq_start=starts)
    i = 0
    for n, L in enumerate(SNAP_LENS):
        for j in range(1, L // every + 1):
            a = starts[n]
            decay = np.exp(g[a:a + j * every].sum(axis=0))  # [H, d_k]
            ref = s0[n] * decay[:, None, :]
            assert _rel(snaps[i], ref) < 1e-13
            i += 1
    assert i == snaps.shape[0]


def test_last_snapshot_is_the_final_state_when_the_interval_divides_the_length():
    q, k, v, beta, g, s0, starts = _snap_case(9)
    _, fin, snaps = oracle.kda_snapshots(q, k, v, g, beta, 16, state0=s0, seq_start=starts)
    # lengths 16 and 96 are multiples of 16: their last snapshots are entries 0 and -1
    assert np.array_equal(snaps[0], fin[2])
    assert np.array_equal(snaps[-1], fin[5])


def test_gdn_forward_is_the_scalar_gate_recurrence():
    """gdn_forward against the Gated DeltaNet update written out with explicit
    d_k x d_k matrices ([K3-explainer] §四), two heads and two sequences."""
    rng = np.random.default_rng(21)
    T, H, dk, dv = 30, 2, 5, 4
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    gs = g[:, :, 0]  # one gate per (token, head)
    starts = [0, 12, 30]
    S0 = rng.standard_normal((2, H, dv, dk)) * 0.3
    out, sT = oracle.gdn_forward(q, k, v, gs, b, state0=S0, seq_start=starts)
    for n in range(2):
        for h in range(H):
            S = S0[n, h].T.copy()
            for t in range(starts[n], starts[n + 1]):
                kt = k[t, h]
                S = np.exp(gs[t, h]) * (np.eye(dk) - b[t, h] * np.outer(kt, kt)) @ S \
                    + b[t, h] * np.outer(kt, v[t, h])
                assert _rel(out[t, h], S.T @ q[t, h]) < 1e-12
            assert _rel(sT[n, h], S.T) < 1e-12
