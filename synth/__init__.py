"""Seeded synthetic inputs for the KDA forward workloads.

This module only draws random numbers and shapes them; it holds none of the
KDA arithmetic.  Both the fp64 oracle (through the tests) and the HIP library
(through the tests, ``bench.py`` and the smoke check) consume what it makes.

Distributions (shared by every workload):
  q, k       ~ N(0, 1), then L2-normalised over the head dimension per
               (token, head) in fp32, then rounded to the workload dtype (RNE);
  v          ~ N(0, 1), rounded to the workload dtype;
  beta       = sigmoid(N(0, 1)), fp32, one per (token, head);
  log_alpha  = -softplus(N(-4, 1)), fp32, one per (token, head, key channel);
  states     ~ N(0, std 0.02) fp32, [N, H, d_v, d_k], when the workload has one.

Draw order inside one generator: lengths (varlen only), q, k, v, beta logits,
gate logits, initial state.  Decode workloads draw the state first, then every
step's q, k, v, beta logits and gate logits as [steps, B, ...] tensors.
Varlen workloads draw the lengths and one sub-seed per sequence from the
master generator, then everything of sequence n from its own generator, so a
single sequence can be regenerated alone.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import torch

__all__ = ["Workload", "WORKLOADS", "prefill_inputs", "decode_inputs",
           "sequence_inputs", "varlen_lengths", "replace"]


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16" for q, k, v, out
    seed: int
    batch: int = 1
    seq_len: int = 0      # dense prefill length (0 for varlen / decode)
    init_std: float = 0.0  # 0 => zero initial state (passed as None)
    n_seqs: int = 0       # varlen: number of packed sequences
    len_range: tuple = (0, 0)  # varlen: inclusive length range
    steps: int = 0        # decode: sequential single-token steps
    draw_block: int = 0   # device draws: tokens per block (0 = the whole sequence at once)
    chunk: int = 64
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", heads=2, head_dim=64, dtype="f32", seed=0, seq_len=256,
                     notes="B=1 H=2 T=256 d=64 fp32, zero initial state"),
    "prefill_4k": Workload("prefill_4k", heads=32, head_dim=128, dtype="bf16", seed=1,
                           seq_len=4096, notes="B=1 H=32 T=4096 d=128 bf16, zero state"),
    "prefill_4k_f32": Workload("prefill_4k_f32", heads=32, head_dim=128, dtype="f32", seed=1,
                               seq_len=4096, notes="B=1 H=32 T=4096 d=128 fp32, zero state"),
    "k3_prefill_32k": Workload("k3_prefill_32k", heads=96, head_dim=128, dtype="bf16",
                               seed=2, seq_len=32768, init_std=0.02,
                               notes="B=1 H=96 T=32768 d=128 bf16, state N(0,0.02)"),
    "varlen_16": Workload("varlen_16", heads=32, head_dim=128, dtype="bf16", seed=3,
                          n_seqs=16, len_range=(1024, 65536), init_std=0.02,
                          notes="16 packed sequences, lengths U[1024,65536], H=32"),
    "long_1m": Workload("long_1m", heads=32, head_dim=128, dtype="bf16", seed=5,
                        seq_len=1 << 20, notes="B=1 H=32 T=1,048,576 d=128 bf16, zero state"),
    "long_1m_h96": Workload("long_1m_h96", heads=96, head_dim=128, dtype="bf16", seed=6,
                            seq_len=1 << 20, draw_block=1 << 16,
                            notes="B=1 H=96 T=1,048,576 d=128 bf16, zero state"),
    "decode_b256": Workload("decode_b256", heads=96, head_dim=128, dtype="bf16", seed=4,
                            batch=256, steps=64, init_std=0.02,
                            notes="B=256 sessions H=96 d=128, 64 single-token steps"),
}


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def _draw(gen, shape, H, d, dtype, init_std, n_states):
    """q, k, v, beta, log_alpha for ``shape`` = leading dims (e.g. (B, T)),
    on the generator's device."""
    dev = gen.device
    q = _unit(torch.randn(*shape, H, d, generator=gen, device=dev)).to(dtype)
    k = _unit(torch.randn(*shape, H, d, generator=gen, device=dev)).to(dtype)
    v = torch.randn(*shape, H, d, generator=gen, device=dev).to(dtype)
    beta = torch.sigmoid(torch.randn(*shape, H, generator=gen, device=dev))
    log_alpha = -torch.nn.functional.softplus(
        torch.randn(*shape, H, d, generator=gen, device=dev) - 4.0)
    state = None
    if init_std > 0:
        state = torch.randn(n_states, H, d, d, generator=gen, device=dev) * init_std
    return q, k, v, beta, log_alpha, state


def varlen_lengths(w: Workload):
    """Sequence lengths and per-sequence sub-seeds of a varlen workload."""
    gen = torch.Generator().manual_seed(w.seed)
    lo, hi = w.len_range
    lengths = torch.randint(lo, hi + 1, (w.n_seqs,), generator=gen)
    subseeds = torch.randint(0, 2**62, (w.n_seqs,), generator=gen)
    return [int(x) for x in lengths], [int(x) for x in subseeds]


def sequence_inputs(w: Workload, n: int):
    """Inputs of packed sequence ``n`` of a varlen workload, drawn on its own."""
    lengths, subseeds = varlen_lengths(w)
    gen = torch.Generator().manual_seed(subseeds[n])
    q, k, v, beta, g, s = _draw(gen, (lengths[n],), w.heads, w.head_dim,
                                _torch_dtype(w.dtype), w.init_std, 1)
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=g, initial_state=s)


def prefill_inputs(w, device=None, **overrides):
    """CPU tensors for one prefill workload.

    ``w`` is a ``Workload`` or a key of ``WORKLOADS``; keyword overrides replace
    Workload fields (e.g. ``seq_len=300`` or ``heads=3``) for smaller cases
    with the same distributions.  ``device`` (dense workloads only) draws the
    tensors there with that device's own generator seeded the same way: same
    distributions and a reproducible draw, but not the CPU draw's numbers (the
    long workloads are too large to draw on the host in reasonable time).

    Dense: q, k, log_alpha [B, T, H, d]; v [B, T, H, d]; beta [B, T, H];
           initial_state [B, H, d, d] or None; cu_seqlens None.
    Varlen: the same with B = 1, T = sum of lengths, initial_state [N, H, d, d]
           and cu_seqlens int32 [N + 1].
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if overrides:
        w = replace(w, **overrides)
    dt = _torch_dtype(w.dtype)
    if device is not None and w.n_seqs:
        raise ValueError("device draws are for dense workloads")
    if w.n_seqs:
        lengths, _ = varlen_lengths(w)
        # Sequences are independent draws: generate them on parallel threads
        # (torch releases the GIL inside randn); the result does not depend on
        # the thread count.
        workers = max(1, min(w.n_seqs, os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            parts = list(pool.map(lambda n: sequence_inputs(w, n), range(w.n_seqs)))
        cat = lambda key: torch.cat([p[key] for p in parts])[None]
        out = {key: cat(key) for key in ("q", "k", "v", "beta", "log_alpha")}
        out["initial_state"] = (torch.cat([p["initial_state"] for p in parts])
                                if w.init_std > 0 else None)
        cu = [0]
        for n in lengths:
            cu.append(cu[-1] + n)
        out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
        out["workload"] = w
        return out
    gen = torch.Generator(device=device or "cpu").manual_seed(w.seed)
    if device is not None and w.draw_block and w.draw_block < w.seq_len:
        return _blocked_device_draw(w, gen, dt)
    q, k, v, beta, g, s = _draw(gen, (w.batch, w.seq_len), w.heads, w.head_dim, dt,
                                w.init_std, w.batch)
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=g, initial_state=s,
                cu_seqlens=None, workload=w)


def _blocked_device_draw(w: Workload, gen, dt):
    """A device draw one block of ``w.draw_block`` tokens at a time (every
    tensor of block 0, then of block 1, ...), so that the fp32 temporaries of a
    very long sequence stay one block in size; the initial state comes last."""
    dev = gen.device
    shape = (w.batch, w.seq_len, w.heads, w.head_dim)
    q = torch.empty(shape, dtype=dt, device=dev)
    k, v = torch.empty_like(q), torch.empty_like(q)
    g = torch.empty(shape, dtype=torch.float32, device=dev)
    beta = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    for t0 in range(0, w.seq_len, w.draw_block):
        t1 = min(w.seq_len, t0 + w.draw_block)
        bq, bk, bv, bb, bg, _ = _draw(gen, (w.batch, t1 - t0), w.heads, w.head_dim, dt, 0.0, 0)
        q[:, t0:t1], k[:, t0:t1], v[:, t0:t1] = bq, bk, bv
        beta[:, t0:t1], g[:, t0:t1] = bb, bg
    s = None
    if w.init_std > 0:
        s = torch.randn(w.batch, w.heads, w.head_dim, w.head_dim, generator=gen,
                        device=dev) * w.init_std
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=g, initial_state=s,
                cu_seqlens=None, workload=w)


def decode_inputs(w="decode_b256", **overrides):
    """CPU tensors for a decode workload: the initial state [B, H, d, d] fp32
    (drawn first), then per step q, k, v [S, B, H, d], beta [S, B, H] and
    log_alpha [S, B, H, d] for S = ``steps`` sequential single-token steps."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if overrides:
        w = replace(w, **overrides)
    gen = torch.Generator().manual_seed(w.seed)
    state = torch.randn(w.batch, w.heads, w.head_dim, w.head_dim, generator=gen) * w.init_std
    q, k, v, beta, g, _ = _draw(gen, (w.steps, w.batch), w.heads, w.head_dim,
                                _torch_dtype(w.dtype), 0.0, 0)
    return dict(state=state, q=q, k=k, v=v, beta=beta, log_alpha=g, workload=w)
