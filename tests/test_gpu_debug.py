"""KDA_DEBUG mode on the GPU, through the C ABI: calls wait for their stream
and check their kernels, packed offsets are checked on the host before any
launch, and results are bitwise those of the default asynchronous mode."""
import numpy as np
import pytest
import torch

import synth
from parity import say

import gated_delta_rule_81_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _packed(lens, seed0=600):
    w = synth.WORKLOADS["varlen_16"]
    parts = [synth.prefill_inputs(w, n_seqs=0, seq_len=n, heads=2, head_dim=64, seed=seed0 + i)
             for i, n in enumerate(lens)]
    cat = lambda key: torch.cat([p[key] for p in parts], dim=1).to(DEV)
    inp = {key: cat(key) for key in ("q", "k", "v", "beta", "log_alpha")}
    inp["initial_state"] = torch.cat([p["initial_state"] for p in parts]).to(DEV)
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]),
                                     dtype=torch.int32, device=DEV)
    return inp


def _fwd(d, cu=None):
    return kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                         d["cu_seqlens"] if cu is None else cu)


def test_debug_mode_same_results(monkeypatch):
    d = _packed([5, 100, 0, 37])
    say("debug mode: prefill, decode, backward")
    o0, f0 = _fwd(d)
    dec = synth.decode_inputs("decode_b256", batch=2, heads=3, head_dim=64, steps=1)
    dd = {k: dec[k][0].to(DEV) for k in ("q", "k", "v", "log_alpha", "beta")}
    s0 = dec["state"].to(DEV)
    s1 = s0.clone()
    y0 = kda.decode_step(*(dd[k] for k in ("q", "k", "v", "log_alpha", "beta")), s0)
    gen = torch.Generator().manual_seed(5)
    d_out = torch.randn(d["q"].shape, generator=gen).to(torch.bfloat16).to(DEV)
    g0 = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d_out, None,
                       d["initial_state"], d["cu_seqlens"])
    torch.cuda.synchronize()
    monkeypatch.setenv("KDA_DEBUG", "1")
    o1, f1 = _fwd(d)
    y1 = kda.decode_step(*(dd[k] for k in ("q", "k", "v", "log_alpha", "beta")), s1)
    g1 = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d_out, None,
                       d["initial_state"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(f0, f1)
    assert torch.equal(y0, y1) and torch.equal(s0, s1)
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "d_initial_state"):
        assert torch.equal(g0[name], g1[name]), name


@pytest.mark.parametrize("cu", [[0, 5, 3, 142], [0, 5, 105, 141], [1, 5, 105, 142]])
def test_debug_mode_rejects_malformed_offsets(monkeypatch, cu):
    """Decreasing offsets, a last offset short of T, a first offset not 0: the
    host check stops the call before any launch."""
    d = _packed([5, 100, 37])  # T = 142
    monkeypatch.setenv("KDA_DEBUG", "1")
    bad = torch.tensor(cu, dtype=torch.int32, device=DEV)
    say("debug mode: malformed offsets", cu)
    with pytest.raises(kda.KdaError, match="KDA_ERR_SHAPE"):
        _fwd(d, bad)
