"""GPU parity of kda_decode_step against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TOL, Worst, f64, max_rel_l2, say, slice_row_errors, state_errors

import gated_delta_rule_81_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_steps(inp, steps, dtype):
    state = inp["state"].to(DEV)
    outs = []
    for s in range(steps):
        args = [inp[key][s].to(DEV) for key in ("q", "k", "v", "log_alpha", "beta")]
        outs.append(kda.decode_step(*args, state).float().cpu())
    torch.cuda.synchronize()
    return torch.stack(outs), state.cpu()


def _oracle_steps(inp, steps, units=None):
    """Oracle over `steps` tokens for the (b, h) pairs in `units` (all if None)."""
    B, H = inp["state"].shape[:2]
    units = [(b, h) for b in range(B) for h in range(H)] if units is None else units
    bs = [u[0] for u in units]
    hs = [u[1] for u in units]
    M = f64(inp["state"][bs, hs])[:, None]  # [U, 1, dv, dk]
    outs = []
    for s in range(steps):
        sel = lambda key: f64(inp[key][s][bs, hs])[:, None]
        o, M = oracle.kda_decode_step(sel("q"), sel("k"), sel("v"), sel("log_alpha"),
                                      f64(inp["beta"][s][bs, hs])[:, None], M)
        outs.append(o[:, 0])
    return np.stack(outs, axis=1), M[:, 0]  # [U, steps, dv], [U, dv, dk]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_small_matches_oracle(dtype, d):
    inp = synth.decode_inputs("decode_b256", batch=3, heads=5, head_dim=d, steps=6, dtype=dtype)
    say("decode small", dtype, d)
    out, state = _run_steps(inp, 6, dtype)
    ref_out, ref_state = _oracle_steps(inp, 6)
    tol = TOL[torch.float32 if dtype == "f32" else torch.bfloat16]
    units = [(b, h) for b in range(3) for h in range(5)]
    e_out = max_rel_l2([(f64(out[:, b, h]), ref_out[i]) for i, (b, h) in enumerate(units)])
    e_st = max_rel_l2([(f64(state[b, h]), ref_state[i]) for i, (b, h) in enumerate(units)])
    print(f"decode {dtype} d={d}: out {e_out:.2e} state {e_st:.2e}")
    assert e_out <= tol and e_st <= tol


def test_decode_full_size_all_units():
    """B=256 sessions, H=96, d=128, 64 sequential steps (the decode workload):
    all 24,576 (session, head) units over all 64 steps, every output row (one
    per step) and every state row against the oracle.  The oracle runs each
    session's 64 tokens as one sequence: a decode step is the recurrence for
    one token, so 64 of them in a row are the recurrence over 64 tokens."""
    w = synth.WORKLOADS["decode_b256"]
    inp = synth.decode_inputs(w)
    say("decode full", w.notes)
    state = inp["state"].to(DEV)
    dev_in = {key: inp[key].to(DEV) for key in ("q", "k", "v", "log_alpha", "beta")}
    outs = torch.empty((w.steps, w.batch, w.heads, w.head_dim), dtype=torch.bfloat16,
                       device=DEV)
    for s in range(w.steps):
        kda.decode_step(*(dev_in[key][s] for key in ("q", "k", "v", "log_alpha", "beta")),
                        state, out=outs[s])
    torch.cuda.synchronize()
    out_gpu = outs.transpose(0, 1).cpu()  # [B, steps, H, d]
    fin_gpu = state.cpu()
    del dev_in, outs, state
    B, S = w.batch, w.steps
    starts = np.arange(B + 1, dtype=np.int64) * S
    # [steps, B, H, ...] -> one sequence per session, [B * steps, h, ...]
    seq = lambda t, h0, h1: f64(t.transpose(0, 1)[:, :, h0:h1].reshape(B * S, h1 - h0,
                                                                        *t.shape[3:]))
    worst = Worst()
    for h0 in range(0, w.heads, 24):
        h1 = min(w.heads, h0 + 24)
        ref_out, ref_st = oracle.kda_forward(
            *(seq(inp[key], h0, h1) for key in ("q", "k", "v", "log_alpha", "beta")),
            state0=f64(inp["state"][:, h0:h1]), seq_start=starts)
        got = f64(out_gpu[:, :, h0:h1].reshape(B * S, h1 - h0, -1))
        worst.add_out(slice_row_errors(got, ref_out, starts))
        worst.add_state(state_errors(f64(fin_gpu[:, h0:h1]), ref_st))
        print(f"  decode full: heads {h0}..{h1 - 1} done ({worst})", flush=True)
    worst.check(torch.bfloat16, "decode full, all units")


def test_decode_steps_equal_chunked_prefill():
    """T decode steps and one chunked prefill over the same T tokens agree."""
    B, H, T, d = 2, 3, 70, 128
    inp = synth.decode_inputs("decode_b256", batch=B, heads=H, head_dim=d, steps=T)
    say("decode vs prefill")
    dev = {key: inp[key].to(DEV) for key in ("q", "k", "v", "log_alpha", "beta")}
    state = inp["state"].to(DEV)
    s0 = state.clone()
    outs = [kda.decode_step(*(dev[key][t] for key in ("q", "k", "v", "log_alpha", "beta")),
                            state) for t in range(T)]
    dec = torch.stack(outs, dim=1).float()  # [B, T, H, d]
    seq = lambda key: dev[key].transpose(0, 1).contiguous()  # [B, T, ...]
    out, fin = kda.chunk_fwd(seq("q"), seq("k"), seq("v"), seq("log_alpha"), seq("beta"), s0)
    torch.cuda.synchronize()
    e = max_rel_l2([(f64(out[b, :, h]), f64(dec[b, :, h])) for b in range(B) for h in range(H)])
    es = max_rel_l2([(f64(fin[b, h]), f64(state[b, h])) for b in range(B) for h in range(H)])
    print(f"decode vs prefill: out {e:.2e} state {es:.2e}")
    assert e <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_decode_zero_batch_is_noop():
    z = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV)
    st = torch.empty((0, 4, 128, 128), device=DEV)
    out = kda.decode_step(z, z, z, torch.empty((0, 4, 128), device=DEV),
                          torch.empty((0, 4), device=DEV), st)
    assert out.shape == (0, 4, 128)
