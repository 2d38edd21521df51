"""fp64 CPU oracle for the Kimi Delta Attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library (``gated_delta_rule_81_amd``) and neither imports the other.

Contents
  * ``kda_forward`` -- ctypes front end of ``kda_oracle.c``: the token-by-token
    recurrence in fp64 (the definition the GPU path must reproduce).
  * ``kda_snapshots`` -- the same recurrence with the state recorded after
    every N tokens of each sequence.
  * ``gdn_forward`` -- the scalar-gate (Gated DeltaNet) special case.
  * ``kda_backward`` -- gradients of ``kda_forward`` with respect to every
    input, token by token in reverse (``kda_oracle.c``).
  * ``forms.projection_forward`` -- a second fp64 witness that builds the
    explicit d_k x d_k transition matrices of the printed KDA update.
  * ``forms.brute_force_exact`` -- exact-rational evaluation through transition
    products, for tiny cases.

Parity pins for every function here live in ``tests/test_oracle_*.py``.

Layout conventions (shared with the library only as a convention, never as code):
  q, k, log_alpha: [T, H, d_k];  v, out: [T, H, d_v];  beta: [T, H];
  states: [N, H, d_v, d_k]  (stored transposed: M = S^T);
  sequences packed along T, sequence n covers tokens [seq_start[n], seq_start[n+1]).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_SO = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` into ``libkda_oracle.so`` with gcc and OpenMP."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def open_library(path: str):
    """Open a compiled oracle at ``path`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_forward.argtypes = [
        ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, dp, dp, dp, dp, dp, dp, dp, dp,
        ctypes.c_int]
    lib.kda_oracle_forward.restype = ctypes.c_int
    lib.kda_oracle_backward.argtypes = [
        ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64] + [dp] * 14 + [ctypes.c_int]
    lib.kda_oracle_backward.restype = ctypes.c_int
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        _lib = open_library(_SO)
    return _lib


def max_threads() -> int:
    """Threads the oracle's OpenMP region uses by default on this host."""
    return int(_load().kda_oracle_max_threads())


def _f64(x, shape=None):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def kda_forward(q, k, v, log_alpha, beta, state0=None, seq_start=None,
                threads: int = 0):
    """Token-by-token KDA forward in fp64.

    Arguments are array-likes (numpy / CPU tensors converted with ``np.asarray``):
      q, k, log_alpha: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H];
      state0: [N, H, d_v, d_k] or None (zeros);
      seq_start: int sequence offsets [N+1] or None (one sequence of length T).
    Returns (out [T, H, d_v], state [N, H, d_v, d_k]) as float64 arrays.
    """
    q = _f64(q)
    if q.ndim != 3:
        raise ValueError("q must be [T, H, d_k]")
    T, H, dk = q.shape
    v = _f64(v)
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, d_v]")
    dv = v.shape[2]
    k = _f64(k, (T, H, dk))
    log_alpha = _f64(log_alpha, (T, H, dk))
    beta = _f64(beta, (T, H))
    if seq_start is None:
        seq_start = [0, T]
    starts = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    N = starts.shape[0] - 1
    if N < 0 or starts[-1] > T or starts[0] < 0 or np.any(np.diff(starts) < 0):
        raise ValueError("seq_start must be non-decreasing within [0, T]")
    s0 = None if state0 is None else _f64(state0, (N, H, dv, dk))
    out = np.zeros((T, H, dv), dtype=np.float64)
    sT = np.zeros((N, H, dv, dk), dtype=np.float64)
    lib = _load()
    rc = lib.kda_oracle_forward(
        N, starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
        _ptr(s0) if s0 is not None else ctypes.POINTER(ctypes.c_double)(),
        _ptr(out), _ptr(sT), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
    return out, sT


def kda_backward(q, k, v, log_alpha, beta, d_out, d_state=None, state0=None,
                 seq_start=None, threads: int = 0):
    """Gradients of ``kda_forward`` in fp64 (``kda_oracle_backward``).

    Inputs as ``kda_forward`` plus d_out [T, H, d_v] (dL/d out) and d_state
    [N, H, d_v, d_k] (dL/d final state) or None (zero).  Returns a dict of
    float64 arrays: dq, dk, dlog_alpha [T, H, d_k]; dv [T, H, d_v];
    dbeta [T, H]; dstate0 [N, H, d_v, d_k] (the initial state's gradient).
    """
    q = _f64(q)
    if q.ndim != 3:
        raise ValueError("q must be [T, H, d_k]")
    T, H, dk = q.shape
    v = _f64(v)
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, d_v]")
    dv = v.shape[2]
    k = _f64(k, (T, H, dk))
    log_alpha = _f64(log_alpha, (T, H, dk))
    beta = _f64(beta, (T, H))
    d_out = _f64(d_out, (T, H, dv))
    if seq_start is None:
        seq_start = [0, T]
    starts = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
    N = starts.shape[0] - 1
    if N < 0 or starts[-1] > T or starts[0] < 0 or np.any(np.diff(starts) < 0):
        raise ValueError("seq_start must be non-decreasing within [0, T]")
    s0 = None if state0 is None else _f64(state0, (N, H, dv, dk))
    ds = None if d_state is None else _f64(d_state, (N, H, dv, dk))
    g = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
         "dlog_alpha": np.zeros((T, H, dk)), "dbeta": np.zeros((T, H)),
         "dstate0": np.zeros((N, H, dv, dk))}
    null = ctypes.POINTER(ctypes.c_double)()
    rc = _load().kda_oracle_backward(
        N, starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
        _ptr(s0) if s0 is not None else null, _ptr(d_out),
        _ptr(ds) if ds is not None else null, _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
        _ptr(g["dlog_alpha"]), _ptr(g["dbeta"]), _ptr(g["dstate0"]), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed with code {rc}")
    return g


def kda_forward_dense(q, k, v, log_alpha, beta, state0=None, threads: int = 0):
    """Dense-batch front end: q, k, log_alpha [B, T, H, d_k]; v [B, T, H, d_v];
    beta [B, T, H]; state0 [B, H, d_v, d_k] or None.
    Returns (out [B, T, H, d_v], state [B, H, d_v, d_k])."""
    q = _f64(q)
    B, T, H, dk = q.shape
    dv = np.shape(v)[-1]
    out, sT = kda_forward(
        q.reshape(B * T, H, dk), _f64(k).reshape(B * T, H, dk),
        _f64(v).reshape(B * T, H, dv), _f64(log_alpha).reshape(B * T, H, dk),
        _f64(beta).reshape(B * T, H), state0,
        seq_start=np.arange(B + 1, dtype=np.int64) * T, threads=threads)
    return out.reshape(B, T, H, dv), sT


def kda_snapshots(q, k, v, log_alpha, beta, every: int, state0=None, seq_start=None,
                  threads: int = 0):
    """The recurrence with its state recorded after every ``every`` tokens of
    each sequence: restartable checkpoints ([K3-memory] §5).

    The definition written out: the state S after the first j * every tokens of
    sequence n, j = 1 .. floor(L_n / every).  It is computed by running the
    token recurrence one segment of ``every`` tokens at a time, each segment
    starting from the state the previous one ended in (all sequences' j-th
    segments in one ``kda_forward`` call).  Same arguments as ``kda_forward``.
    Returns (out [T, H, d_v], final state [N, H, d_v, d_k], snapshots
    [S, H, d_v, d_k]) with S = sum_n floor(L_n / every), sequences in order and
    each sequence's snapshots in token order.
    """
    every = int(every)
    if every <= 0:
        raise ValueError("every must be positive")
    q = _f64(q)
    T, H, dk = q.shape
    k, v, log_alpha, beta = _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    dv = v.shape[2]
    if seq_start is None:
        seq_start = [0, T]
    starts = np.asarray(seq_start, dtype=np.int64)
    N = starts.shape[0] - 1
    lengths = starts[1:] - starts[:-1]
    counts = lengths // every
    base = np.concatenate([[0], np.cumsum(counts)])
    snaps = np.zeros((int(base[-1]), H, dv, dk), dtype=np.float64)
    out = np.zeros((T, H, dv), dtype=np.float64)
    state = (np.zeros((N, H, dv, dk)) if state0 is None else _f64(state0, (N, H, dv, dk)).copy())
    nseg = int(np.max((lengths + every - 1) // every)) if N > 0 else 0
    for j in range(nseg):
        # segment j of every sequence: tokens [start + j*every, min(start + (j+1)*every, end))
        lo = np.minimum(starts[:-1] + j * every, starts[1:])
        hi = np.minimum(starts[:-1] + (j + 1) * every, starts[1:])
        idx = np.concatenate([np.arange(a, b) for a, b in zip(lo, hi)]).astype(np.int64)
        seg_start = np.concatenate([[0], np.cumsum(hi - lo)])
        o, state = kda_forward(q[idx], k[idx], v[idx], log_alpha[idx], beta[idx], state,
                               seq_start=seg_start, threads=threads)
        out[idx] = o
        for n in range(N):
            if j < counts[n]:
                snaps[base[n] + j] = state[n]
    return out, state, snaps


def gdn_forward(q, k, v, log_alpha, beta, state0=None, seq_start=None, threads: int = 0):
    """Gated DeltaNet in fp64: one gate per (token, head) shared by every key
    channel, S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
    ([K3-explainer] §四, the scalar-gate form KDA refines).  With Diag(alpha_t)
    = alpha_t I this is the KDA recurrence with the gate repeated over the
    channels, so ``kda_forward`` computes it.  log_alpha: [T, H]; everything
    else as ``kda_forward``."""
    q = _f64(q)
    T, H, dk = q.shape
    g = _f64(log_alpha, (T, H))
    return kda_forward(q, k, v, np.repeat(g[:, :, None], dk, axis=2), beta, state0=state0,
                       seq_start=seq_start, threads=threads)


def kda_decode_step(q, k, v, log_alpha, beta, state, threads: int = 0):
    """One decode token per session: q, k, log_alpha [B, H, d_k]; v [B, H, d_v];
    beta [B, H]; state [B, H, d_v, d_k].  A decode step is the recurrence run
    for a single token, so this is ``kda_forward`` with B sequences of length 1.
    Returns (out [B, H, d_v], new_state [B, H, d_v, d_k])."""
    q = _f64(q)
    B = q.shape[0]
    out, sT = kda_forward(q, k, v, log_alpha, beta, state,
                          seq_start=np.arange(B + 1, dtype=np.int64),
                          threads=threads)
    return out, sT
