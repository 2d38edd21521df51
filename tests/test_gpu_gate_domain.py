"""The whole gate domain alpha in [0, 1]^{d_k} ([K3-explainer] §四) on the GPU,
through the C ABI, against the fp64 oracle.

The chunked prefill factorises a chunk's products with e^{+-(decay inside a
16-token block)}; a chunk in which some channel decays by more than 2^-100 over
a block (or has alpha = 0, i.e. log_alpha = -inf) is stepped token by token
instead, in fp32.  These cases drive both sides of that switch: -inf gates at
scattered tokens and channels, long runs of strong decay (log_alpha = -8, -20),
mixed chunks, the scalar-gate entry point, packed sequences, snapshots, the
segmented prefill and the decode step, and the fast path just inside its range
(log_alpha = -4: a 16-token block decays by 2^-92)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, check_prefill_full, f64, max_rel_l2, say

import gated_delta_rule_81_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NEG_INF = float("-inf")


def _case(dtype, d, T=300, heads=3, batch=2, seed=41):
    w = "k3_prefill_32k" if dtype == "bf16" else "tiny"
    return synth.prefill_inputs(w, seq_len=T, heads=heads, head_dim=d, batch=batch,
                                init_std=0.02, seed=seed)


def _run(inp, **kw):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                             d["initial_state"], d.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return out.cpu(), fin.cpu()


def _gates(g, kind):
    """Put a pattern of out-of-range gates into log_alpha [B, T, H, d] (in place)."""
    rng = np.random.default_rng(7)
    B, T, H, D = g.shape
    if kind == "inf_scattered":  # alpha = 0 on random (token, head, channel) entries
        m = torch.from_numpy(rng.random(g.shape) < 0.01)
        g[m] = NEG_INF
    elif kind == "inf_tokens":  # alpha = 0 on every channel of a few tokens
        for t in (0, 5, 33, 64, 200, T - 1):
            if t < T:
                g[:, t] = NEG_INF
    elif kind == "minus8_runs":
        g[:, 40:140] = -8.0
        g[:, 230:260, :, :7] = -8.0
    elif kind == "minus20":
        g[:] = -20.0
    elif kind == "mixed":  # a few channels at -20 in some chunks, -inf in one
        g[:, 70:90, :, 3:5] = -20.0
        if T > 150:
            g[:, 150, H - 1, 100 % D] = NEG_INF
        g[:, 260:300, :, :2] = -12.0
    elif kind == "edge_minus4":  # inside the factorised range (2^-92 per block)
        g[:] = -4.0
    else:
        raise ValueError(kind)
    return g


KINDS = ["inf_scattered", "inf_tokens", "minus8_runs", "minus20", "mixed", "edge_minus4"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_gate_domain_prefill(kind, dtype, d):
    inp = _case(dtype, d)
    _gates(inp["log_alpha"], kind)
    say("gate domain prefill", kind, dtype, d)
    out, fin = _run(inp)
    assert torch.isfinite(out.float()).all() and torch.isfinite(fin).all()
    check_prefill_full(inp, out, fin, label=f"gate domain {kind} {dtype} d={d}")


@pytest.mark.parametrize("kind", ["inf_tokens", "minus20", "mixed"])
def test_gate_domain_scalar_gate(kind):
    inp = _case("bf16", 128)
    g = inp["log_alpha"][..., 0].clone()
    if kind == "inf_tokens":
        g[:, [3, 31, 32, 200]] = NEG_INF
    elif kind == "minus20":
        g[:] = -20.0
    else:
        g[:, 40:100] = -9.0
        g[:, 250] = NEG_INF
    gpu = dict(inp)
    gpu["log_alpha"] = g.contiguous()
    ref = dict(inp)
    ref["log_alpha"] = g[..., None].expand_as(inp["log_alpha"]).contiguous()
    say("gate domain scalar gate", kind)
    out, fin = _run(gpu, scalar_gate=True)
    check_prefill_full(ref, out, fin, label=f"gate domain scalar {kind}")


def test_gate_domain_packed():
    lens = [0, 1, 45, 64, 130, 7, 300]
    w = synth.WORKLOADS["varlen_16"]
    parts = [synth.prefill_inputs(w, n_seqs=0, seq_len=n, heads=2, seed=300 + i)
             for i, n in enumerate(lens)]
    for i, p in enumerate(parts):
        if p["q"].shape[1]:
            _gates(p["log_alpha"], ["inf_tokens", "minus8_runs", "mixed"][i % 3]
                   if p["q"].shape[1] > 1 else "minus20")
    cat = lambda key: torch.cat([p[key] for p in parts], dim=1)
    inp = {key: cat(key) for key in ("q", "k", "v", "beta", "log_alpha")}
    inp["initial_state"] = torch.cat([p["initial_state"] for p in parts])
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    say("gate domain packed", lens)
    out, fin = _run(inp)
    check_prefill_full(inp, out, fin, label="gate domain packed")


def test_gate_domain_snapshots_and_segmented():
    inp = _case("bf16", 128, T=1000, batch=1)
    _gates(inp["log_alpha"], "mixed")
    inp["log_alpha"][:, 500:560] = -15.0
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = [d[key] for key in ("q", "k", "v", "log_alpha", "beta")]
    say("gate domain snapshots and segmented")
    out, fin, snaps = kda.chunk_fwd_snapshots(*args, 96, d["initial_state"])
    out_s, fin_s = kda.chunk_fwd_segmented(*args, 4, d["initial_state"])
    torch.cuda.synchronize()
    check_prefill_full(inp, out.cpu(), fin.cpu(), label="gate domain snapshots: out")
    check_prefill_full(inp, out_s.cpu(), fin_s.cpu(), label="gate domain segmented")
    flat = lambda key: f64(inp[key][0])
    _, _, ref = oracle.kda_snapshots(flat("q"), flat("k"), flat("v"), flat("log_alpha"),
                                     flat("beta"), 96, state0=f64(inp["initial_state"]))
    got = f64(snaps.cpu())
    err = max_rel_l2([(got[i, h], ref[i, h]) for i in range(got.shape[0]) for h in range(3)])
    print(f"gate domain snapshots: {err:.2e}")
    assert err <= TOL[torch.bfloat16]


def test_gate_domain_decode():
    dec = synth.decode_inputs("decode_b256", batch=4, heads=3, steps=6)
    dec["log_alpha"][1, :, :, :9] = NEG_INF
    dec["log_alpha"][3] = -30.0
    dec["log_alpha"][4, 2] = NEG_INF
    state = dec["state"].to(DEV)
    M = f64(dec["state"])
    say("gate domain decode")
    worst = 0.0
    for s in range(6):
        args = [dec[k][s] for k in ("q", "k", "v", "log_alpha", "beta")]
        o = kda.decode_step(*(a.to(DEV) for a in args), state)
        o_ref, M = oracle.kda_decode_step(*(f64(a) for a in args), M)
        worst = max(worst, max_rel_l2([(f64(o.cpu())[b, h], o_ref[b, h])
                                       for b in range(4) for h in range(3)]))
    torch.cuda.synchronize()
    es = max_rel_l2([(f64(state.cpu())[b, h], M[b, h]) for b in range(4) for h in range(3)])
    print(f"gate domain decode: out {worst:.2e} state {es:.2e}")
    assert worst <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_gate_domain_in_place_state_and_selective_fixup():
    """Out-of-range gates in one head of one sequence only, with the final
    state written over the initial state: the marked unit is recomputed from
    its original initial state, the other units keep the fast kernel's
    results (bitwise equal to a run without the far gates there), and the
    far results are deterministic."""
    inp = _case("bf16", 128, T=200, heads=4, batch=3)
    clean = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    inp["log_alpha"][1, 50:90, 2] = -30.0
    inp["log_alpha"][1, 120, 2, 7] = NEG_INF
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = [d[key] for key in ("q", "k", "v", "log_alpha", "beta")]
    say("gate domain in place, one far unit")
    state = d["initial_state"].clone()
    out, fin = kda.chunk_fwd(*args, state, final_state=state)
    out2, fin2 = kda.chunk_fwd(*args, d["initial_state"])
    c = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in clean.items()}
    out_c, fin_c = kda.chunk_fwd(*(c[key] for key in ("q", "k", "v", "log_alpha", "beta")),
                                 c["initial_state"])
    torch.cuda.synchronize()
    assert fin.data_ptr() == state.data_ptr()
    assert torch.equal(out, out2) and torch.equal(fin, fin2)
    check_prefill_full(inp, out.cpu(), fin.cpu(), label="gate domain in place")
    for b in range(3):
        for h in range(4):
            if (b, h) != (1, 2):
                assert torch.equal(out[b, :, h], out_c[b, :, h]) and torch.equal(fin[b, h], fin_c[b, h])


# ---------------------------------------------------------------- backward
# kda_chunk_bwd marks the (sequence, head) units whose gates leave the chunked
# backward's range (a 16-token block decaying beyond 2^-100 in a channel,
# -inf or NaN gates) and recomputes all their gradients token by token in fp32
# after the chunked kernels; the other units keep the chunked results.
from test_gpu_backward import compare, loss_grads, oracle_grads, packed_parts, run_gpu  # noqa: E402

BWD_KINDS = KINDS + ["one_unit"]


def _bwd_gates(g, kind):
    if kind == "one_unit":  # a single -inf entry: only unit (0, 1) leaves the range
        g[0, 37, 1, 5] = NEG_INF
        return g
    return _gates(g, kind)


@pytest.mark.parametrize("kind", BWD_KINDS)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_gate_domain_backward(kind, dtype, d):
    inp = _case(dtype, d, T=200)
    _bwd_gates(inp["log_alpha"], kind)
    d_out, d_fin = loss_grads(inp, 5)
    say("gate domain backward", kind, dtype, d)
    g = run_gpu(inp, d_out, d_fin)
    for name, t in g.items():
        assert torch.isfinite(t.float()).all(), name
    compare(inp, g, oracle_grads(inp, d_out, d_fin), label=f"bwd gate domain {kind} {dtype} d={d}")


def test_gate_domain_backward_selective():
    """Only unit (sequence 1, head 2) leaves the range: the other units'
    gradients are bitwise those of a run without the far gates, and repeated
    runs are bitwise equal."""
    inp = _case("bf16", 128, T=150, heads=4, batch=3)
    clean = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    inp["log_alpha"][1, 20:60, 2] = -30.0
    inp["log_alpha"][1, 100, 2, 9] = NEG_INF
    d_out, d_fin = loss_grads(inp, 8)
    say("gate domain backward, one far unit")
    g = run_gpu(inp, d_out, d_fin)
    g2 = run_gpu(inp, d_out, d_fin)
    gc = run_gpu(clean, d_out, d_fin)
    for name in g:
        assert torch.equal(g[name], g2[name]), name
    compare(inp, g, oracle_grads(inp, d_out, d_fin), label="bwd gate domain one far unit")
    for b in range(3):
        for h in range(4):
            if (b, h) == (1, 2):
                continue
            for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
                assert torch.equal(g[name][b, :, h], gc[name][b, :, h]), (name, b, h)
            assert torch.equal(g["d_initial_state"][b, h], gc["d_initial_state"][b, h])


def test_gate_domain_backward_packed():
    lens = [0, 1, 16, 45, 130, 7, 260]
    w = synth.WORKLOADS["varlen_16"]

    def make(i, n):
        p = synth.prefill_inputs(w, n_seqs=0, seq_len=n, heads=2, seed=500 + i)
        if n > 1:
            _gates(p["log_alpha"], ["inf_tokens", "minus8_runs", "mixed", "edge_minus4"][i % 4])
        elif n == 1:
            p["log_alpha"][:] = NEG_INF
        return p

    inp = packed_parts(lens, make)
    d_out, d_fin = loss_grads(inp, 9)
    say("gate domain backward packed", lens)
    g = run_gpu(inp, d_out, d_fin)
    compare(inp, g, oracle_grads(inp, d_out, d_fin), label="bwd gate domain packed")
    assert torch.equal(g["d_initial_state"][0].cpu(), d_fin[0])
