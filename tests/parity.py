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
