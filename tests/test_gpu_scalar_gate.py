"""GPU parity of the scalar-gate (Gated DeltaNet) entry points against the fp64
oracle, through the C ABI.

The scalar gate of a (token, head) is taken from the seeded per-channel gates
(their first channel), so its distribution is the workloads' log_alpha
distribution.  The oracle is the KDA recurrence with that gate repeated over the
key channels, which ``oracle.gdn_forward`` and its pins tie to the Gated
DeltaNet update ([K3-explainer] §四).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, check_prefill_full, f64, max_rel_l2, say

import gated_delta_rule_81_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def scalar_case(inp):
    """(GPU inputs with log_alpha [B, T, H], oracle inputs with it broadcast)."""
    g = inp["log_alpha"][..., 0].contiguous()
    gpu = dict(inp)
    gpu["log_alpha"] = g
    ref = dict(inp)
    ref["log_alpha"] = g[..., None].expand_as(inp["log_alpha"]).contiguous()
    return gpu, ref


def run(inp):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                             d["initial_state"], d.get("cu_seqlens"), scalar_gate=True)
    torch.cuda.synchronize()
    return out, fin


def check(ref, out, fin, label=""):
    """Every (sequence, head) slice and every row against the oracle (``ref``
    carries the scalar gate repeated over the channels)."""
    check_prefill_full(ref, out.cpu(), fin.cpu(), label=label)


def test_scalar_gate_tiny_fp32():
    gpu, ref = scalar_case(synth.prefill_inputs("tiny", init_std=0.02))
    say("scalar gate tiny fp32")
    out, fin = run(gpu)
    check(ref, out, fin, label="scalar gate tiny fp32")


@pytest.mark.parametrize("T", [1, 31, 65, 333])
@pytest.mark.parametrize("d", [64, 128])
def test_scalar_gate_bf16_ragged(T, d):
    gpu, ref = scalar_case(synth.prefill_inputs("k3_prefill_32k", seq_len=T, heads=3,
                                                head_dim=d, batch=2))
    say("scalar gate bf16", T, d)
    out, fin = run(gpu)
    check(ref, out, fin, label=f"scalar gate bf16 T={T} d={d}")


def test_scalar_gate_varlen_small():
    lens = [0, 1, 63, 64, 65, 130, 7, 0, 200]
    w = synth.WORKLOADS["varlen_16"]
    parts = [synth.prefill_inputs(w, n_seqs=0, seq_len=n, heads=4, seed=500 + i)
             for i, n in enumerate(lens)]
    cat = lambda key: torch.cat([p[key] for p in parts], dim=1)
    inp = {key: cat(key) for key in ("q", "k", "v", "beta", "log_alpha")}
    inp["initial_state"] = torch.cat([p["initial_state"] for p in parts])
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    gpu, ref = scalar_case(inp)
    say("scalar gate varlen", lens)
    out, fin = run(gpu)
    check(ref, out, fin, label="scalar gate varlen")


def test_scalar_gate_agrees_with_the_channel_gate_kernel():
    """The same gates given per channel to kda_chunk_fwd: both kernels within
    the bf16 bound of each other (they differ only in rounding order)."""
    gpu, ref = scalar_case(synth.prefill_inputs("k3_prefill_32k", seq_len=500, heads=4))
    say("scalar gate vs channel gate")
    out_s, fin_s = run(gpu)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in ref.items()}
    out_c, fin_c = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                 d["initial_state"])
    torch.cuda.synchronize()
    e = max_rel_l2([(f64(out_s[0, :, h].cpu()), f64(out_c[0, :, h].cpu())) for h in range(4)])
    es = max_rel_l2([(f64(fin_s[0, h].cpu()), f64(fin_c[0, h].cpu())) for h in range(4)])
    print(f"scalar vs channel gate kernels: out {e:.2e} state {es:.2e}")
    assert e <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_scalar_gate_k3_prefill_32k_all_heads():
    """The 32K x 96-head launch with scalar gates: all heads, every row."""
    gpu, ref = scalar_case(synth.prefill_inputs("k3_prefill_32k"))
    say("scalar gate k3 32k")
    out, fin = run(gpu)
    del gpu
    check(ref, out, fin, label="scalar gate k3 32k")


def test_scalar_gate_decode_steps():
    """16 decode steps of 8 sessions x 4 heads (d=128, bf16) with scalar gates."""
    w = synth.replace(synth.WORKLOADS["decode_b256"], batch=8, heads=4, steps=16)
    dec = synth.decode_inputs(w)
    state = dec["state"].to(DEV)
    ref_state = f64(dec["state"])
    say("scalar gate decode")
    worst = 0.0
    for t in range(w.steps):
        g = dec["log_alpha"][t][..., 0].contiguous()  # [B, H]
        out = kda.decode_step(dec["q"][t].to(DEV), dec["k"][t].to(DEV), dec["v"][t].to(DEV),
                              g.to(DEV), dec["beta"][t].to(DEV), state, scalar_gate=True)
        torch.cuda.synchronize()
        o_ref, ref_state = oracle.kda_decode_step(
            f64(dec["q"][t]), f64(dec["k"][t]), f64(dec["v"][t]),
            np.repeat(f64(g)[:, :, None], w.head_dim, axis=2), f64(dec["beta"][t]), ref_state)
        o = f64(out.cpu())
        worst = max(worst, max_rel_l2([(o[b, h], o_ref[b, h]) for b in range(w.batch)
                                       for h in range(w.heads)]))
    s = f64(state.cpu())
    es = max_rel_l2([(s[b, h], ref_state[b, h]) for b in range(w.batch) for h in range(w.heads)])
    print(f"scalar gate decode: out {worst:.2e} state {es:.2e}")
    assert worst <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]
