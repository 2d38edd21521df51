"""PyTorch front end of the KDA library: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/kda.h); this module checks tensor metadata, allocates outputs with
torch (device memory) and passes raw pointers plus torch's current stream.

Pages cited (by title):
  [K3-explainer]  lshu.cn news 263999, the Kimi K3 explainer (§四: the update;
                  §六.2: a chunk's updates as one transition matrix).
  [K3-memory]     "Kimi K3 Changed the Memory Math for Agentic AI Forever" (§3:
                  the [batch, heads, value_dim, key_dim] state layout).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._lib import KDA_DTYPE_BF16, KDA_DTYPE_F32, check, lib

_DTYPES = {torch.float32: KDA_DTYPE_F32, torch.bfloat16: KDA_DTYPE_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _expect(t, name, dtype, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, *, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
              scalar_gate: bool = False
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA prefill (``kda_chunk_fwd``; with ``scalar_gate=True``,
    ``kda_chunk_fwd_scalar_gate``: log_alpha is [B, T, H], one Gated DeltaNet
    gate per token and head applied to every key channel).

    q, k, log_alpha: [B, T, H, d_k]; v: [B, T, H, d_v]; beta: [B, T, H];
    initial_state: [N, H, d_v, d_k] fp32 or None (zeros); cu_seqlens: int32
    [N + 1] on the device for packed sequences (then B must be 1), else None
    and N = B.  q, k, v share one dtype (float32 or bfloat16); gates and
    states are float32.  Returns (out [B, T, H, d_v], final_state or None).
    ``final_state`` may be passed in (and may be ``initial_state`` itself).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _expect(q, "q", q.dtype, (B, T, H, dk), dev)
    _expect(k, "k", q.dtype, (B, T, H, dk), dev)
    _expect(v, "v", q.dtype, (B, T, H, dv), dev)
    _expect(log_alpha, "log_alpha", torch.float32,
            (B, T, H) if scalar_gate else (B, T, H, dk), dev)
    _expect(beta, "beta", torch.float32, (B, T, H), dev)
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be 1-D")
        _expect(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.shape, dev)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    _expect(initial_state, "initial_state", torch.float32, (N, H, dv, dk), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _expect(out, "out", q.dtype, (B, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    _expect(final_state, "final_state", torch.float32, (N, H, dv, dk), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    name = "kda_chunk_fwd_scalar_gate" if scalar_gate else "kda_chunk_fwd"
    rc = getattr(lib(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
        _ptr(cu_seqlens), _ptr(out), _ptr(final_state), B, T, H, dk, dv,
        N if cu_seqlens is not None else 0, _DTYPES[q.dtype], stream)
    check(rc, name)
    return out, final_state


def chunk_fwd_snapshots(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        log_alpha: torch.Tensor, beta: torch.Tensor, snapshot_every: int,
                        initial_state: Optional[torch.Tensor] = None,
                        cu_seqlens: Optional[torch.Tensor] = None, *,
                        num_snapshots: Optional[int] = None,
                        out: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None,
                        snapshots: Optional[torch.Tensor] = None,
                        output_final_state: bool = True
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """``chunk_fwd`` that also returns the state after every ``snapshot_every``
    tokens of each sequence (``kda_chunk_fwd_snapshots``; [K3-memory] §5).

    Returns (out, final_state, snapshots [S, H, d_v, d_k] fp32): the snapshots
    of all sequences in sequence order, each sequence's in token order, S =
    sum over sequences of floor(length / snapshot_every).  For packed input
    the count needs the lengths: pass ``num_snapshots``, or it is computed from
    a host copy of ``cu_seqlens`` (a device synchronisation).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    every = int(snapshot_every)
    if every <= 0:
        raise ValueError("snapshot_every must be positive")
    _expect(q, "q", q.dtype, (B, T, H, dk), dev)
    _expect(k, "k", q.dtype, (B, T, H, dk), dev)
    _expect(v, "v", q.dtype, (B, T, H, dv), dev)
    _expect(log_alpha, "log_alpha", torch.float32, (B, T, H, dk), dev)
    _expect(beta, "beta", torch.float32, (B, T, H), dev)
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be 1-D")
        _expect(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.shape, dev)
        N = cu_seqlens.shape[0] - 1
        if num_snapshots is None:
            lengths = cu_seqlens.to("cpu", torch.int64)
            num_snapshots = int(((lengths[1:] - lengths[:-1]) // every).sum())
    else:
        N = B
        if num_snapshots is None:
            num_snapshots = B * (T // every)
    _expect(initial_state, "initial_state", torch.float32, (N, H, dv, dk), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _expect(out, "out", q.dtype, (B, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    _expect(final_state, "final_state", torch.float32, (N, H, dv, dk), dev)
    if snapshots is None:
        snapshots = torch.empty((num_snapshots, H, dv, dk), dtype=torch.float32, device=dev)
    _expect(snapshots, "snapshots", torch.float32, (num_snapshots, H, dv, dk), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().kda_chunk_fwd_snapshots(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
        _ptr(cu_seqlens), _ptr(out), _ptr(final_state), _ptr(snapshots), every, num_snapshots,
        B, T, H, dk, dv, N if cu_seqlens is not None else 0, _DTYPES[q.dtype], stream)
    check(rc, "kda_chunk_fwd_snapshots")
    return out, final_state, snapshots


def segmented_workspace_size(seq_len: int, num_heads: int, head_dim: int,
                             num_segments: int) -> int:
    """Bytes of workspace ``chunk_fwd_segmented`` needs
    (``kda_chunk_fwd_segmented_workspace_size``)."""
    n = lib().kda_chunk_fwd_segmented_workspace_size(seq_len, num_heads, head_dim, num_segments)
    if n < 0:
        raise ValueError(f"invalid sizes seq_len={seq_len} num_heads={num_heads} "
                         f"head_dim={head_dim} num_segments={num_segments}")
    return int(n)


def chunk_fwd_segmented(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        log_alpha: torch.Tensor, beta: torch.Tensor, num_segments: int,
                        initial_state: Optional[torch.Tensor] = None, *,
                        workspace: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None,
                        output_final_state: bool = True
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd`` of one long sequence (B = 1, no cu_seqlens) split into
    ``num_segments`` segments that run in parallel (``kda_chunk_fwd_segmented``):
    per-segment state maps, a fold over the segments, then every segment again
    from its entering state ([K3-explainer] §六.2, the chunk transition).

    ``workspace`` is a uint8 device tensor of at least
    ``segmented_workspace_size(T, H, d_k, num_segments)`` bytes (allocated here
    when None).  Returns (out [1, T, H, d_v], final_state [1, H, d_v, d_k] or None).
    """
    if q.dim() != 4 or q.shape[0] != 1:
        raise ValueError("q must be [1, T, H, d_k]")
    _, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _expect(q, "q", q.dtype, (1, T, H, dk), dev)
    _expect(k, "k", q.dtype, (1, T, H, dk), dev)
    _expect(v, "v", q.dtype, (1, T, H, dv), dev)
    _expect(log_alpha, "log_alpha", torch.float32, (1, T, H, dk), dev)
    _expect(beta, "beta", torch.float32, (1, T, H), dev)
    _expect(initial_state, "initial_state", torch.float32, (1, H, dv, dk), dev)
    need = segmented_workspace_size(T, H, dk, int(num_segments))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _expect(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    if out is None:
        out = torch.empty((1, T, H, dv), dtype=q.dtype, device=dev)
    _expect(out, "out", q.dtype, (1, T, H, dv), dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((1, H, dv, dk), dtype=torch.float32, device=dev)
    _expect(final_state, "final_state", torch.float32, (1, H, dv, dk), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().kda_chunk_fwd_segmented(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
        _ptr(out), _ptr(final_state), T, H, dk, dv, int(num_segments), _DTYPES[q.dtype],
        _ptr(workspace), workspace.numel(), stream)
    check(rc, "kda_chunk_fwd_segmented")
    return out, final_state


def chunk_fwd_segmented_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                log_alpha: torch.Tensor, beta: torch.Tensor, num_segments: int,
                                initial_state: Optional[torch.Tensor], out: torch.Tensor,
                                final_state: Optional[torch.Tensor]) -> None:
    """``chunk_fwd_segmented`` into caller-given outputs with the library's
    fixed scratch instead of a workspace (``kda_chunk_fwd_segmented_noalloc``):
    this call allocates no device memory, neither here nor in the library.
    Requests needing more than ``KDA_SCRATCH_BYTES`` raise KDA_ERR_SCRATCH.
    Calls that may overlap in time on one GPU must not be issued (they share
    its one scratch buffer)."""
    if q.dim() != 4 or q.shape[0] != 1:
        raise ValueError("q must be [1, T, H, d_k]")
    _, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _expect(q, "q", q.dtype, (1, T, H, dk), dev)
    _expect(k, "k", q.dtype, (1, T, H, dk), dev)
    _expect(v, "v", q.dtype, (1, T, H, dv), dev)
    _expect(log_alpha, "log_alpha", torch.float32, (1, T, H, dk), dev)
    _expect(beta, "beta", torch.float32, (1, T, H), dev)
    _expect(initial_state, "initial_state", torch.float32, (1, H, dv, dk), dev)
    if out is None:
        raise ValueError("out must be given (this call allocates nothing)")
    _expect(out, "out", q.dtype, (1, T, H, dv), dev)
    _expect(final_state, "final_state", torch.float32, (1, H, dv, dk), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().kda_chunk_fwd_segmented_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
        _ptr(out), _ptr(final_state), T, H, dk, dv, int(num_segments), _DTYPES[q.dtype], stream)
    check(rc, "kda_chunk_fwd_segmented_noalloc")


def bwd_workspace_size(total_tokens: int, num_seqs: int, num_heads: int, head_dim: int) -> int:
    """Bytes of workspace ``chunk_bwd`` needs (``kda_chunk_bwd_workspace_size``)."""
    n = lib().kda_chunk_bwd_workspace_size(total_tokens, num_seqs, num_heads, head_dim)
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
              beta: torch.Tensor, d_out: torch.Tensor,
              d_final_state: Optional[torch.Tensor] = None,
              initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, *,
              workspace: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
              output_initial_state_grad: bool = True) -> dict:
    """Gradients of ``chunk_fwd`` (``kda_chunk_bwd``): given dL/d out and
    dL/d final_state (None = zero), returns a dict with dq, dk, dv (dtype of
    q), dlog_alpha, dbeta (fp32) and d_initial_state (fp32, or None when
    ``output_initial_state_grad`` is False).  Inputs as for ``chunk_fwd``;
    ``grads`` may hold preallocated outputs under the same names, and
    ``workspace`` a uint8 device tensor of ``bwd_workspace_size`` bytes.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t, name, dt, shp in ((q, "q", q.dtype, (B, T, H, dk)), (k, "k", q.dtype, (B, T, H, dk)),
                             (v, "v", q.dtype, (B, T, H, dv)),
                             (log_alpha, "log_alpha", torch.float32, (B, T, H, dk)),
                             (beta, "beta", torch.float32, (B, T, H)),
                             (d_out, "d_out", q.dtype, (B, T, H, dv))):
        _expect(t, name, dt, shp, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be 1-D")
        _expect(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.shape, dev)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    _expect(initial_state, "initial_state", torch.float32, (N, H, dv, dk), dev)
    _expect(d_final_state, "d_final_state", torch.float32, (N, H, dv, dk), dev)
    g = dict(grads or {})
    shapes = {"dq": (q.dtype, (B, T, H, dk)), "dk": (q.dtype, (B, T, H, dk)),
              "dv": (q.dtype, (B, T, H, dv)), "dlog_alpha": (torch.float32, (B, T, H, dk)),
              "dbeta": (torch.float32, (B, T, H)),
              "d_initial_state": (torch.float32, (N, H, dv, dk))}
    for name, (dt, shp) in shapes.items():
        if name == "d_initial_state" and not output_initial_state_grad and name not in g:
            g[name] = None
            continue
        if g.get(name) is None:
            g[name] = torch.empty(shp, dtype=dt, device=dev)
        _expect(g[name], name, dt, shp, dev)
    need = bwd_workspace_size(B * T, N, H, dk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _expect(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().kda_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(initial_state),
        _ptr(cu_seqlens), _ptr(d_out), _ptr(d_final_state), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["dbeta"]), _ptr(g["d_initial_state"]),
        B, T, H, dk, dv, N if cu_seqlens is not None else 0, _DTYPES[q.dtype],
        _ptr(workspace), workspace.numel(), stream)
    check(rc, "kda_chunk_bwd")
    return g


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                scalar_gate: bool = False) -> torch.Tensor:
    """One decode token per session (``kda_decode_step``), state updated in place.
    With ``scalar_gate=True`` (``kda_decode_step_scalar_gate``) log_alpha is
    [B, H]: one Gated DeltaNet gate per session and head.

    q, k, log_alpha: [B, H, d_k]; v: [B, H, d_v]; beta: [B, H];
    state: [B, H, d_v, d_k] fp32.  Returns out [B, H, d_v] (dtype of q).
    """
    if q.dim() != 3:
        raise ValueError("q must be [B, H, d_k]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    _expect(k, "k", q.dtype, (B, H, dk), dev)
    _expect(v, "v", q.dtype, (B, H, dv), dev)
    _expect(log_alpha, "log_alpha", torch.float32, (B, H) if scalar_gate else (B, H, dk), dev)
    _expect(beta, "beta", torch.float32, (B, H), dev)
    _expect(state, "state", torch.float32, (B, H, dv, dk), dev)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _expect(out, "out", q.dtype, (B, H, dv), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    name = "kda_decode_step_scalar_gate" if scalar_gate else "kda_decode_step"
    rc = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                              _ptr(state), _ptr(out), B, H, dk, dv, _DTYPES[q.dtype], stream)
    check(rc, name)
    return out
