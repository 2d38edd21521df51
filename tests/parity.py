"""Helpers for GPU-vs-oracle parity tests (imported by the gpu test modules).

Metric: per (sequence, head) slice, relative L2 error ||x - x*|| / ||x*|| of the
outputs (T_n x d_v) and of the final state (d_v x d_k); a test passes when the
maximum over slices is within its tolerance.  A slice whose reference norm is
below 1e-12 of the largest slice norm is judged by absolute L2 error instead.
Tolerances: 1e-4 for fp32 q/k/v, 2e-2 for bf16 q/k/v.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(*msg):
    """Name the case on stdout before a GPU step (flushed, survives a crash)."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def seq_starts(inp):
    q = inp["q"]
    B, T = q.shape[:2]
    if inp.get("cu_seqlens") is not None:
        return [int(x) for x in inp["cu_seqlens"]]
    return [b * T for b in range(B + 1)]


def oracle_prefill(inp, seqs=None, heads=None, threads=0):
    """Oracle outputs for a subset of sequences and heads.

    Returns (starts_sub, out [T_sub, h, d_v], state [n, h, d_v, d_k]) where the
    selected sequences are packed in the given order."""
    q = inp["q"]
    B, T, H, D = q.shape
    starts = seq_starts(inp)
    N = len(starts) - 1
    seqs = list(range(N)) if seqs is None else list(seqs)
    heads = list(range(H)) if heads is None else list(heads)
    flat = lambda key: inp[key].reshape(B * T, *inp[key].shape[2:])
    idx = np.concatenate([np.arange(starts[n], starts[n + 1]) for n in seqs] + [[]]).astype(np.int64)
    sub = {}
    for key in ("q", "k", "v", "log_alpha"):
        sub[key] = f64(flat(key)[idx][:, heads])
    sub["beta"] = f64(flat("beta")[idx][:, heads])
    s0 = inp.get("initial_state")
    state0 = None if s0 is None else f64(s0[seqs][:, heads])
    lens = [starts[n + 1] - starts[n] for n in seqs]
    st = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    out, sT = oracle.kda_forward(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"],
                                 state0=state0, seq_start=st, threads=threads)
    return st, out, sT, idx


def max_rel_l2(pairs):
    """Max over (got, ref) pairs of the slice error defined in the module doc."""
    norms = [np.linalg.norm(r) for _, r in pairs]
    big = max(norms) if norms else 0.0
    worst = 0.0
    for (g, r), n in zip(pairs, norms):
        d = np.linalg.norm(np.asarray(g, np.float64) - r)
        err = d / n if n > 1e-12 * big and n > 0 else d
        worst = max(worst, err)
    return worst


def compare_prefill(inp, out_gpu, state_gpu, seqs=None, heads=None, threads=0):
    """Returns (max out error, max state error) over the selected slices."""
    q = inp["q"]
    B, T, H, D = q.shape
    starts = seq_starts(inp)
    N = len(starts) - 1
    seqs = list(range(N)) if seqs is None else list(seqs)
    heads = list(range(H)) if heads is None else list(heads)
    st, out_ref, s_ref, idx = oracle_prefill(inp, seqs, heads, threads)
    og = f64(out_gpu.reshape(B * T, H, -1)[torch.as_tensor(idx)][:, heads]) if len(idx) else \
        np.zeros((0, len(heads), out_ref.shape[-1]))
    out_pairs, st_pairs = [], []
    for i, n in enumerate(seqs):
        for j, h in enumerate(heads):
            out_pairs.append((og[st[i]:st[i + 1], j], out_ref[st[i]:st[i + 1], j]))
            if state_gpu is not None:
                st_pairs.append((f64(state_gpu[n, h]), s_ref[i, j]))
    e_out = max_rel_l2([p for p in out_pairs if p[1].size])
    e_st = max_rel_l2(st_pairs) if st_pairs else 0.0
    return e_out, e_st


# ---------------------------------------------------------------- full-size checks
# Per-row bound.  One relative L2 per (sequence, head) slice cannot see a single
# wrong token row of a long slice (one row of 32,768 moves it by ~0.5%), so the
# full-size checks also bound every row: token rows of the outputs, value rows of
# the states.  A row's error is ||x_r - x*_r|| / max(||x*_r||, rms), where rms is
# the slice's root-mean-square row norm: relative for ordinary rows, and relative
# to the slice's typical row for rows whose reference is near zero (whose error,
# which scales with |q| |S| rather than with |o|, would otherwise look huge).
# A wrong row (a zero row, another token's row) has an error near 1.  The bound is
# the slice bound times ROW_FACTOR: the rounding error of a row is a sum over d
# independent terms, so across the ~3e6 rows of a workload its norm spreads about
# the slice's mean by a chi distribution with d degrees of freedom, whose maximum
# over 3e6 draws stays below ~1.5x the mean; the factor 2 leaves room above that.
ROW_FACTOR = 2.0
ROW_TOL = {dt: ROW_FACTOR * t for dt, t in TOL.items()}
# Rows of one element (the backward's dbeta, one per token and head) have no
# averaging over d: the maximum of ~3e6 near-Gaussian errors sits ~5.5 standard
# deviations out, so their bound is the slice bound times 6.
DBETA_ROW_TOL = {dt: 6.0 * t for dt, t in TOL.items()}


def slice_row_errors(got, ref, starts):
    """Errors of packed token rows.

    got, ref: [T, h, d] arrays (tokens packed along axis 0, sequence n covering
    rows starts[n] .. starts[n+1]); returns (max slice rel-L2, max row error)
    over every non-empty (sequence, head) slice, with the slice metric of
    ``max_rel_l2`` (absolute below 1e-12 of the largest slice norm) and the row
    metric described above."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    T = ref.shape[0]
    if T == 0:
        return 0.0, 0.0
    e2 = np.sum((got - ref) ** 2, axis=-1)  # [T, h]
    r2 = np.sum(ref ** 2, axis=-1)
    zero = np.zeros((1,) + e2.shape[1:])
    ce = np.concatenate([zero, np.cumsum(e2, axis=0)])
    cr = np.concatenate([zero, np.cumsum(r2, axis=0)])
    st = np.asarray(starts, np.int64)
    lens = st[1:] - st[:-1]
    keep = lens > 0
    E = (ce[st[1:]] - ce[st[:-1]])[keep]  # [n, h]
    R = np.maximum(cr[st[1:]] - cr[st[:-1]], 0.0)[keep]
    nR = np.sqrt(R)
    big = nR.max() if nR.size else 0.0
    rel = np.where((nR > 1e-12 * big) & (nR > 0), np.sqrt(E) / np.where(nR > 0, nR, 1.0),
                   np.sqrt(E))
    slice_err = float(rel.max()) if rel.size else 0.0
    # row floor: the slice's mean squared row norm, broadcast to its rows
    seq_of_row = np.repeat(np.arange(len(lens)), lens)
    ms = (cr[st[1:]] - cr[st[:-1]]) / np.maximum(lens, 1)[:, None]  # [N, h]
    floor = ms[seq_of_row]
    den = np.maximum(r2, floor)
    row = np.where(den > 0, np.sqrt(e2 / np.where(den > 0, den, 1.0)), np.sqrt(e2))
    return slice_err, float(row.max())


def state_errors(got, ref):
    """(max slice rel-L2, max row error) of states [N, h, d_v, d_k]: each
    (sequence, head) state is a slice, its value rows are the rows."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    N, h, dv, dk = ref.shape
    # every state is a sequence of dv rows
    g = got.reshape(N * h, dv, dk).transpose(1, 0, 2).reshape(dv, N * h, dk)
    r = ref.reshape(N * h, dv, dk).transpose(1, 0, 2).reshape(dv, N * h, dk)
    # rows of slice u are g[:, u]: treat the slices as "heads" of one sequence
    return slice_row_errors(g, r, [0, dv])


class Worst:
    """Running maxima of slice and row errors for outputs and states."""

    def __init__(self):
        self.out = self.out_row = self.state = self.state_row = 0.0

    def add_out(self, pair):
        self.out, self.out_row = max(self.out, pair[0]), max(self.out_row, pair[1])

    def add_state(self, pair):
        self.state, self.state_row = max(self.state, pair[0]), max(self.state_row, pair[1])

    def __str__(self):
        return (f"out {self.out:.2e} (row {self.out_row:.2e}) "
                f"state {self.state:.2e} (row {self.state_row:.2e})")

    def check(self, dtype, label=""):
        tol, rtol = TOL[dtype], ROW_TOL[dtype]
        print(f"{label}: {self} (tol {tol}, row tol {rtol})", flush=True)
        assert self.out <= tol and self.state <= tol, (label, str(self))
        assert self.out_row <= rtol and self.state_row <= rtol, (label, str(self))


def _heads_f64(t, B, T, h0, h1):
    """[B, T, H, ...] tensor -> float64 numpy [B*T, h1-h0, ...]."""
    x = t.reshape(B * T, *t.shape[2:])[:, h0:h1]
    return x.to(torch.float32).numpy().astype(np.float64)


def check_prefill_full(inp, out_gpu, fin_gpu, group=16, oracle_fn=None, threads=0, label=""):
    """Every (sequence, head) slice and every row of a prefill's outputs and
    final states against the oracle, heads taken ``group`` at a time to bound
    host memory.  out_gpu / fin_gpu are CPU tensors (fin may be None).
    ``oracle_fn(q, k, v, g, b, state0, seq_start)`` defaults to
    ``oracle.kda_forward``; log_alpha may be [B, T, H] (scalar gates)."""
    q = inp["q"]
    B, T, H, D = q.shape
    starts = seq_starts(inp)
    run = oracle_fn or (lambda *a, **kw: oracle.kda_forward(*a, **kw))
    w = Worst()
    s0 = inp.get("initial_state")
    for h0 in range(0, H, group):
        h1 = min(H, h0 + group)
        args = [_heads_f64(inp[key], B, T, h0, h1) for key in ("q", "k", "v", "log_alpha")]
        b = _heads_f64(inp["beta"], B, T, h0, h1)
        st0 = None if s0 is None else f64(s0[:, h0:h1])
        ref_out, ref_st = run(*args, b, state0=st0, seq_start=starts, threads=threads)
        del args, b
        w.add_out(slice_row_errors(_heads_f64(out_gpu, B, T, h0, h1), ref_out, starts))
        if fin_gpu is not None:
            w.add_state(state_errors(f64(fin_gpu[:, h0:h1]), ref_st))
        if H > group:  # progress of long comparisons
            print(f"  {label}: heads {h0}..{h1 - 1} done ({w})", flush=True)
    w.check(q.dtype, label)
    return w
