"""The 1M-token prefill at K3's 96 heads ([Kimi-Linear], Figure 7 at 1M
context; [K3-memory] §3, 96 heads of d = 128), through the C ABI: one
B=1 H=96 T=1,048,576 d=128 bf16 sequence drawn on the device (about 150 GB of
inputs and outputs in HBM), two heads checked over all tokens against the
oracle, and the segmented entry point, which cannot gain at 96 heads, running
the plain prefill (bitwise equal)."""
import pytest
import torch

import synth
from parity import check_prefill_full, say

import gated_delta_rule_81_amd as kda

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_long_1m_h96_two_heads_and_segmented_fallback():
    w = synth.WORKLOADS["long_1m_h96"]
    say("long_1m_h96: drawing on the device", w.notes)
    d = synth.prefill_inputs(w, device=DEV)
    args = [d[key] for key in ("q", "k", "v", "log_alpha", "beta")]
    say("long_1m_h96: kda_chunk_fwd")
    out, fin = kda.chunk_fwd(*args, None)
    torch.cuda.synchronize()
    heads = [0, 95]
    sub = {key: d[key][:, :, heads].cpu() for key in ("q", "k", "v", "log_alpha", "beta")}
    sub["initial_state"] = None
    sub["cu_seqlens"] = None
    out_h = out[:, :, heads].cpu()
    fin_h = fin[:, heads].cpu()
    say("long_1m_h96: kda_chunk_fwd_segmented G=4 (falls back to the plain prefill)")
    ws = torch.empty(kda.segmented_workspace_size(w.seq_len, w.heads, w.head_dim, 4),
                     dtype=torch.uint8, device=DEV)
    out2 = torch.empty_like(out)
    fin2 = torch.empty_like(fin)
    kda.chunk_fwd_segmented(*args, 4, None, workspace=ws, out=out2, final_state=fin2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(fin2, fin)
    del d, args, out, out2, fin, fin2, ws
    say("long_1m_h96: oracle on heads", heads)
    check_prefill_full(sub, out_h, fin_h, label="long_1m_h96 heads 0 and 95")
