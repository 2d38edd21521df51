"""fp32 q/k/v at d_k = d_v = 128 through every prefill entry point, on the GPU
through the C ABI, against the fp64 oracle (bound 1e-4).  The library runs
this size as the token recurrence itself in fp32 (the chunked kernel's fp32
operand sets do not fit one CU's LDS at d = 128)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, check_prefill_full, f64, max_rel_l2, say

import gated_delta_rule_81_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inp(T, heads=3, batch=2, seed=51, **kw):
    return synth.prefill_inputs("tiny", seq_len=T, heads=heads, head_dim=128, batch=batch,
                                init_std=0.02, seed=seed, **kw)


def _dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _run(inp, **kw):
    d = _dev(inp)
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                             d["initial_state"], d.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return out.cpu(), fin.cpu()


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100, 333])
def test_fp32_d128_dense(T):
    inp = _inp(T)
    assert inp["q"].dtype == torch.float32
    say("fp32 d128 dense", T)
    out, fin = _run(inp)
    check_prefill_full(inp, out, fin, label=f"fp32 d=128 T={T}")


def test_fp32_d128_packed_and_empty():
    lens = [0, 1, 63, 64, 65, 0, 200]
    parts = [_inp(n, heads=2, batch=1, seed=60 + i) for i, n in enumerate(lens)]
    cat = lambda key: torch.cat([p[key] for p in parts], dim=1)
    inp = {key: cat(key) for key in ("q", "k", "v", "beta", "log_alpha")}
    inp["initial_state"] = torch.cat([p["initial_state"] for p in parts])
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    say("fp32 d128 packed", lens)
    out, fin = _run(inp)
    check_prefill_full(inp, out, fin, label="fp32 d=128 packed")
    for n in (0, 5):
        assert torch.equal(fin[n], inp["initial_state"][n])


def test_fp32_d128_layer_all_heads():
    """B=1 H=32 T=4096 d=128 in fp32: every head and row."""
    inp = synth.prefill_inputs("prefill_4k", dtype="f32")
    assert inp["q"].dtype == torch.float32
    say("fp32 d128 4K layer")
    out, fin = _run(inp)
    check_prefill_full(inp, out, fin, label="fp32 d=128 4K x 32 heads")


def test_fp32_d128_gate_domain_and_in_place():
    inp = _inp(300)
    g = inp["log_alpha"]
    g[:, 40:90] = -20.0
    g[:, 150, :, 3] = float("-inf")
    g[:, 200:210, 1] = float("-inf")
    d = _dev(inp)
    say("fp32 d128 gate domain, in place")
    state = d["initial_state"].clone()
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state,
                             final_state=state)
    torch.cuda.synchronize()
    check_prefill_full(inp, out.cpu(), fin.cpu(), label="fp32 d=128 gate domain")


def test_fp32_d128_null_states():
    inp = _inp(70, heads=2, batch=1)
    d = _dev(inp)
    say("fp32 d128 null states")
    o1, f1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None)
    o2, f2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                           torch.zeros_like(d["initial_state"]))
    o3, f3 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None,
                           output_final_state=False)
    torch.cuda.synchronize()
    assert f3 is None and torch.equal(o1, o2) and torch.equal(f1, f2) and torch.equal(o1, o3)


def test_fp32_d128_scalar_gate():
    inp = _inp(150)
    g = inp["log_alpha"][..., 0].contiguous()
    ref = dict(inp)
    ref["log_alpha"] = g[..., None].expand_as(inp["log_alpha"]).contiguous()
    gpu = dict(inp)
    gpu["log_alpha"] = g
    say("fp32 d128 scalar gate")
    out, fin = _run(gpu, scalar_gate=True)
    check_prefill_full(ref, out, fin, label="fp32 d=128 scalar gate")


def test_fp32_d128_snapshots():
    inp = _inp(300, batch=1)
    d = _dev(inp)
    say("fp32 d128 snapshots")
    out, fin, snaps = kda.chunk_fwd_snapshots(d["q"], d["k"], d["v"], d["log_alpha"],
                                              d["beta"], 96, d["initial_state"])
    out0, fin0 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(out, out0) and torch.equal(fin, fin0)
    flat = lambda key: f64(inp[key][0])
    _, _, ref = oracle.kda_snapshots(flat("q"), flat("k"), flat("v"), flat("log_alpha"),
                                     flat("beta"), 96, state0=f64(inp["initial_state"]))
    got = f64(snaps.cpu())
    assert got.shape == ref.shape
    err = max_rel_l2([(got[i, h], ref[i, h]) for i in range(got.shape[0]) for h in range(3)])
    print(f"fp32 d=128 snapshots: {err:.2e}")
    assert err <= TOL[torch.float32]


@pytest.mark.parametrize("G", [2, 5])
def test_fp32_d128_segmented(G):
    inp = _inp(1000, batch=1)
    d = _dev(inp)
    args = [d[key] for key in ("q", "k", "v", "log_alpha", "beta")]
    say("fp32 d128 segmented", G)
    out, fin = kda.chunk_fwd_segmented(*args, G, d["initial_state"])
    torch.cuda.synchronize()
    check_prefill_full(inp, out.cpu(), fin.cpu(), label=f"fp32 d=128 segmented G={G}")
