"""GPU test of kda_chunk_fwd_segmented_noalloc, the segmented prefill with the
library's fixed scratch instead of a caller workspace, through the C ABI: its
outputs and final states equal kda_chunk_fwd_segmented's bitwise (same
kernels, same order) on two calls in a row, the second smaller than the first,
and both lie within the parity bound of the fp64 oracle."""
import numpy as np
import pytest
import torch

import synth
from parity import check_prefill_full, say

import gated_delta_rule_81_amd as kda
from gated_delta_rule_81_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(seq_len, heads, head_dim, dtype, seed):
    w = "k3_prefill_32k" if dtype == "bf16" else "tiny"
    return synth.prefill_inputs(w, seq_len=seq_len, heads=heads, head_dim=head_dim,
                                init_std=0.02, seed=seed)


def _both(inp, G):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = [d[k] for k in ("q", "k", "v", "log_alpha", "beta")]
    ref_out, ref_fin = kda.chunk_fwd_segmented(*args, G, d["initial_state"])
    out = torch.empty_like(ref_out)
    fin = torch.empty_like(ref_fin)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    kda.chunk_fwd_segmented_noalloc(*args, G, d["initial_state"], out, fin)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return out, fin, ref_out, ref_fin


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(4000, 4, 128, "bf16", 31, 4),  # 4 segments of 1,024 tokens, 4 MiB of scratch
             (700, 2, 64, "f32", 32, 3)]      # then a smaller call: 3 segments
    for T, H, D, dt, seed, G in cases:
        inp = _case(T, H, D, dt, seed)
        need = kda.segmented_workspace_size(T, H, D, G)
        assert 0 < need <= _lib.KDA_SCRATCH_BYTES
        say("noalloc segmented", T, H, D, dt, "G", G, "scratch bytes", need)
        out, fin, ref_out, ref_fin = _both(inp, G)
        assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)
        check_prefill_full(inp, out.cpu(), fin.cpu(), label=f"noalloc T={T} H={H} d={D} {dt}")


def test_noalloc_rejects_requests_beyond_the_scratch():
    T, H, D = 1 << 14, 64, 128  # 8 segments x 64 heads: 128 MiB of maps and states
    assert kda.segmented_workspace_size(T, H, D, 8) > _lib.KDA_SCRATCH_BYTES
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device=DEV)
    q = z(1, T, H, D)
    say("noalloc beyond the scratch")
    with pytest.raises(kda.KdaError, match="KDA_ERR_SCRATCH"):
        kda.chunk_fwd_segmented_noalloc(q, q.clone(), q.clone(), z(1, T, H, D, dt=torch.float32),
                                        z(1, T, H, dt=torch.float32), 8, None, q.clone(), None)
