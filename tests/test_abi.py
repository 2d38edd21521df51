"""The C ABI library loads, exports what include/kda.h declares, and rejects bad
arguments on the host before any device work (no GPU needed).

Pointers passed here are fake, 16-byte-aligned integers: validation never
dereferences them, and every case below stops at a host-side check.
"""
import ctypes
import os
import re

import pytest

from gated_delta_rule_81_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, DEVICE, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -8
BF16, F32 = 1, 0


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["kda_abi_version", "kda_chunk_bwd", "kda_chunk_bwd_workspace_size",
         "kda_chunk_fwd", "kda_chunk_fwd_scalar_gate",
         "kda_chunk_fwd_segmented", "kda_chunk_fwd_segmented_noalloc",
         "kda_chunk_fwd_segmented_workspace_size",
         "kda_chunk_fwd_snapshots", "kda_decode_step", "kda_decode_step_scalar_gate",
         "kda_status_string"])


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(handle, name), name
    assert set(_lib.SIGNATURES) == set(declared_functions())


def test_abi_version_and_status_strings():
    L = _lib.lib()
    assert L.kda_abi_version() == 7
    for code in range(-8, 1):
        assert L.kda_status_string(code).decode() not in ("", "unknown status")
    assert L.kda_status_string(12345) == b"unknown status"


# ---------------------------------------------------------------- chunk_fwd
GB = 1 << 30


class Buf:
    """Fake device buffers at far-apart aligned addresses."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self):
        p = self.next
        self.next += 64 * GB
        return p


def chunk_args(**kw):
    b = Buf()
    args = dict(q=b(), k=b(), v=b(), log_alpha=b(), beta=b(), initial_state=b(),
                cu_seqlens=None, out=b(), final_state=b(), batch=2, seq_len=100,
                num_heads=3, head_dim_k=128, head_dim_v=128, num_seqs=0, dtype=BF16,
                stream=None)
    args.update(kw)
    return args


def call_chunk(**kw):
    a = chunk_args(**kw)
    return _lib.lib().kda_chunk_fwd(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"],
        a["cu_seqlens"], a["out"], a["final_state"], a["batch"], a["seq_len"],
        a["num_heads"], a["head_dim_k"], a["head_dim_v"], a["num_seqs"], a["dtype"],
        a["stream"])


@pytest.mark.parametrize("name", ["q", "k", "v", "log_alpha", "beta", "out"])
def test_chunk_null_required_pointer(name):
    assert call_chunk(**{name: None}) == NULL


def test_chunk_optional_pointers_may_be_null():
    # with no GPU in this container the call gets as far as the device check
    rc = call_chunk(initial_state=None, final_state=None)
    assert rc in (DEVICE, OK)


@pytest.mark.parametrize("kw", [dict(batch=-1), dict(seq_len=-5), dict(num_heads=-1),
                                dict(head_dim_k=0), dict(head_dim_v=-128)])
def test_chunk_bad_sizes(kw):
    assert call_chunk(**kw) == SHAPE


def test_chunk_packed_requires_batch_one():
    b = Buf()
    assert call_chunk(cu_seqlens=b(), batch=2, num_seqs=2) == SHAPE
    assert call_chunk(cu_seqlens=b(), batch=1, num_seqs=-1) == SHAPE


def test_chunk_token_count_must_fit_int32():
    assert call_chunk(batch=70000, seq_len=70000) == SHAPE


@pytest.mark.parametrize("kw", [dict(head_dim_k=128, head_dim_v=64), dict(head_dim_k=96,
                                head_dim_v=96), dict(head_dim_k=256, head_dim_v=256),
                                dict(dtype=7)])
def test_chunk_unsupported(kw):
    assert call_chunk(**kw) == UNSUP


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_chunk_supported_set(d, dtype):
    """d_k = d_v in {64, 128} with fp32 or bf16 q/k/v: valid calls reach the
    device check (no GPU here) or run."""
    assert call_chunk(dtype=dtype, head_dim_k=d, head_dim_v=d) in (DEVICE, OK)


def test_chunk_head_count_bound_for_32bit_offsets():
    # 64 tokens of log_alpha (H * d fp32 each) must span less than 2^31 bytes
    assert call_chunk(num_heads=65536, batch=1, seq_len=1) == UNSUP
    assert call_chunk(num_heads=65535, batch=1, seq_len=1) in (DEVICE, OK)


@pytest.mark.parametrize("name", ["q", "k", "v", "log_alpha", "initial_state", "out",
                                  "final_state"])
def test_chunk_misaligned(name):
    a = chunk_args()
    assert call_chunk(**{name: a[name] + 8}) == ALIGN


def test_chunk_scalar_arrays_need_four_bytes():
    a = chunk_args()
    assert call_chunk(beta=a["beta"] + 2) == ALIGN
    assert call_chunk(beta=a["beta"] + 4) in (DEVICE, OK)
    assert call_chunk(cu_seqlens=(1 << 50) + 2, batch=1, num_seqs=3) == ALIGN


def test_chunk_output_overlapping_input_is_rejected():
    a = chunk_args()
    assert call_chunk(out=a["q"] + 256) == ALIAS
    assert call_chunk(out=a["log_alpha"]) == ALIAS
    assert call_chunk(final_state=a["v"] + 4096) == ALIAS
    assert call_chunk(out=a["final_state"]) == ALIAS


def test_chunk_in_place_state_is_allowed():
    a = chunk_args()
    assert call_chunk(final_state=a["initial_state"]) in (DEVICE, OK)
    # a partial overlap of the two states is not
    assert call_chunk(final_state=a["initial_state"] + 1024) == ALIAS


def test_chunk_empty_work_returns_ok_without_device():
    assert call_chunk(batch=0) == OK
    assert call_chunk(num_heads=0) == OK
    b = Buf()
    assert call_chunk(cu_seqlens=b(), batch=1, num_seqs=0, seq_len=0) == OK


def test_chunk_zero_tokens_allows_null_inputs():
    # T = 0 still copies initial -> final state, so it reaches the device check
    rc = call_chunk(seq_len=0, q=None, k=None, v=None, log_alpha=None, beta=None, out=None)
    assert rc in (DEVICE, OK)


# ---------------------------------------------------------------- chunk_fwd_snapshots
def call_snap(snapshots="auto", snapshot_every=64, num_snapshots=None, **kw):
    a = chunk_args(**kw)
    if snapshots == "auto":
        snapshots = (1 << 50)
    if num_snapshots is None:
        num_snapshots = a["batch"] * (a["seq_len"] // snapshot_every) if snapshot_every > 0 else 1
    return _lib.lib().kda_chunk_fwd_snapshots(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"],
        a["cu_seqlens"], a["out"], a["final_state"], snapshots, snapshot_every, num_snapshots,
        a["batch"], a["seq_len"], a["num_heads"], a["head_dim_k"], a["head_dim_v"],
        a["num_seqs"], a["dtype"], a["stream"])


def test_snapshots_valid_call_reaches_the_device_check():
    assert call_snap() in (DEVICE, OK)
    assert call_snap(snapshot_every=32, seq_len=100) in (DEVICE, OK)


@pytest.mark.parametrize("every", [0, -32])
def test_snapshots_interval_must_be_positive(every):
    assert call_snap(snapshot_every=every, num_snapshots=1) == SHAPE


@pytest.mark.parametrize("every", [1, 48, 100])
def test_snapshots_interval_must_be_a_chunk_multiple(every):
    assert call_snap(snapshot_every=every) == UNSUP


def test_snapshots_dense_capacity_is_checked():
    # batch 2 x floor(200 / 64) = 6 entries needed
    assert call_snap(seq_len=200, num_snapshots=5) == SHAPE
    assert call_snap(seq_len=200, num_snapshots=6) in (DEVICE, OK)
    assert call_snap(seq_len=200, num_snapshots=-1) == SHAPE
    # fewer tokens than one interval: no entry needed, the buffer may be NULL
    assert call_snap(seq_len=63, snapshots=None, num_snapshots=0) in (DEVICE, OK)


def test_snapshots_packed_capacity_is_not_checked_on_host():
    b = Buf()
    assert call_snap(cu_seqlens=b(), batch=1, num_seqs=3, seq_len=500,
                     num_snapshots=1) in (DEVICE, OK)


def test_snapshots_null_buffer_with_entries():
    assert call_snap(snapshots=None, num_snapshots=6, seq_len=200) == NULL


def test_snapshots_misaligned_and_aliased():
    a = chunk_args()
    assert call_snap(snapshots=(1 << 50) + 8) == ALIGN
    assert call_snap(snapshots=a["out"]) == ALIAS
    assert call_snap(snapshots=a["final_state"] + 1024) == ALIAS
    assert call_snap(snapshots=a["q"]) == ALIAS
    assert call_snap(snapshots=a["initial_state"]) == ALIAS


def test_snapshots_share_the_chunk_fwd_checks():
    assert call_snap(q=None) == NULL
    assert call_snap(head_dim_k=96, head_dim_v=96) == UNSUP
    assert call_snap(dtype=F32) in (DEVICE, OK)
    assert call_snap(batch=0) == OK


# ---------------------------------------------------------------- chunk_fwd_segmented
def seg_size(T, H, D, G):
    return _lib.lib().kda_chunk_fwd_segmented_workspace_size(T, H, D, G)


def test_segmented_workspace_size():
    st = lambda n, H, D: n * H * D * D * 4
    # 1000 tokens in 4 requested segments: 256-token segments, 4 of them
    assert seg_size(1000, 3, 128, 4) == 256 + 4 * st(4, 3, 128)
    # 100 tokens in 8: segments of one chunk (32 tokens), 4 of them
    assert seg_size(100, 2, 64, 8) == 256 + 4 * st(4, 2, 64)
    # 65 offsets need 260 bytes, padded to 512
    assert seg_size(64 * 32, 1, 64, 64) == 512 + 4 * st(64, 1, 64)
    assert seg_size(0, 3, 128, 4) == 256
    assert seg_size(5000, 0, 128, 4) == 256
    for bad in [(-1, 3, 128, 4), (100, -1, 128, 4), (100, 3, 96, 4), (100, 3, 128, 0)]:
        assert seg_size(*bad) == -1


WS = 1 << 52


def call_seg(num_segments=4, workspace=WS, workspace_bytes=None, **kw):
    kw.setdefault("batch", 1)
    kw.setdefault("seq_len", 1000)
    a = chunk_args(**kw)
    if workspace_bytes is None:
        workspace_bytes = max(seg_size(a["seq_len"], a["num_heads"], a["head_dim_k"],
                                       max(num_segments, 1)), 0)
    return _lib.lib().kda_chunk_fwd_segmented(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"], a["out"],
        a["final_state"], a["seq_len"], a["num_heads"], a["head_dim_k"], a["head_dim_v"],
        num_segments, a["dtype"], workspace, workspace_bytes, a["stream"])


def test_segmented_valid_call_reaches_the_device_check():
    assert call_seg() in (DEVICE, OK)
    assert call_seg(initial_state=None, final_state=None) in (DEVICE, OK)


def test_segmented_checks():
    a = chunk_args()
    assert call_seg(num_segments=0) == SHAPE
    assert call_seg(num_segments=-2) == SHAPE
    assert call_seg(q=None) == NULL
    assert call_seg(seq_len=-1) == SHAPE
    assert call_seg(head_dim_k=96, head_dim_v=96) == UNSUP
    assert call_seg(workspace=None) == NULL
    assert call_seg(workspace_bytes=seg_size(1000, 3, 128, 4) - 1) == SHAPE
    assert call_seg(workspace_bytes=-1) == SHAPE
    assert call_seg(workspace=WS + 128) == ALIGN
    assert call_seg(workspace=a["out"]) == ALIAS
    assert call_seg(workspace=a["q"] - 1024) == ALIAS
    assert call_seg(workspace=a["initial_state"] + 4096) == ALIAS


def test_segmented_one_segment_needs_no_workspace():
    # a single segment (or a sequence of at most one chunk per segment) is the
    # plain prefill: the workspace is never touched
    assert call_seg(num_segments=1, workspace=None, workspace_bytes=0) in (DEVICE, OK)
    assert call_seg(seq_len=32, num_segments=8, workspace=None, workspace_bytes=0) in (DEVICE, OK)
    assert call_seg(seq_len=0, workspace=None, workspace_bytes=0, q=None, k=None, v=None,
                    log_alpha=None, beta=None, out=None) in (DEVICE, OK)
    assert call_seg(num_heads=0, workspace=None, workspace_bytes=0) == OK


def call_seg_noalloc(num_segments=4, **kw):
    kw.setdefault("batch", 1)
    kw.setdefault("seq_len", 1000)
    a = chunk_args(**kw)
    return _lib.lib().kda_chunk_fwd_segmented_noalloc(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"], a["out"],
        a["final_state"], a["seq_len"], a["num_heads"], a["head_dim_k"], a["head_dim_v"],
        num_segments, a["dtype"], a["stream"])


def test_segmented_noalloc_checks():
    """The fixed-scratch entry point: kda_chunk_fwd_segmented's checks, then the
    scratch limit, all before any device call."""
    assert _lib.KDA_SCRATCH_BYTES == 64 << 20
    assert call_seg_noalloc() in (DEVICE, OK)
    assert call_seg_noalloc(num_segments=0) == SHAPE
    assert call_seg_noalloc(q=None) == NULL
    assert call_seg_noalloc(head_dim_k=96, head_dim_v=96) == UNSUP
    a = chunk_args()
    assert call_seg_noalloc(out=a["q"]) == ALIAS
    # 1M tokens x 32 heads at d = 128: 4 segments need 32 MiB (fits), 16 need
    # 128 MiB (does not)
    big = dict(seq_len=1 << 20, num_heads=32)
    assert seg_size(1 << 20, 32, 128, 4) <= _lib.KDA_SCRATCH_BYTES
    assert call_seg_noalloc(4, **big) in (DEVICE, OK)
    assert seg_size(1 << 20, 32, 128, 16) > _lib.KDA_SCRATCH_BYTES
    assert call_seg_noalloc(16, **big) == SCRATCH
    # one segment is the plain prefill: no scratch, whatever the size
    assert call_seg_noalloc(1, seq_len=1 << 20, num_heads=96) in (DEVICE, OK)
    assert call_seg_noalloc(4, seq_len=1 << 20, num_heads=96) == SCRATCH
    assert call_seg_noalloc(num_heads=0) == OK


# ---------------------------------------------------------------- chunk_bwd
def test_bwd_workspace_size():
    f = _lib.lib().kda_chunk_bwd_workspace_size
    # two regions of one fp32 state per 16-token slot and head, then 16 flag
    # words per (sequence, head) marking gates outside the chunked range
    assert f(200, 2, 3, 128) == 2 * (200 // 16 + 2 + 1) * 3 * 128 * 128 * 4 + 16 * 2 * 3 * 4
    assert f(0, 0, 3, 64) == 2 * 1 * 3 * 64 * 64 * 4
    for bad in [(-1, 1, 1, 64), (10, -1, 1, 64), (10, 1, -1, 64), (10, 1, 1, 96)]:
        assert f(*bad) == -1


def call_bwd(workspace="auto", workspace_bytes=None, **kw):
    b = Buf()
    b.next = 1 << 47  # clear of the buffers chunk_args hands out
    grads = dict(d_out=b(), d_final_state=b(), dq=b(), dk=b(), dv=b(), dlog_alpha=b(),
                 dbeta=b(), d_initial_state=b())
    for key in list(grads):
        if key in kw:
            grads[key] = kw.pop(key)
    a = chunk_args(**kw)
    N = a["num_seqs"] if a["cu_seqlens"] else a["batch"]
    if workspace == "auto":
        workspace = 1 << 52
    if workspace_bytes is None:
        workspace_bytes = max(0, _lib.lib().kda_chunk_bwd_workspace_size(
            a["batch"] * a["seq_len"], N, a["num_heads"], a["head_dim_k"]))
    return _lib.lib().kda_chunk_bwd(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"], a["cu_seqlens"],
        grads["d_out"], grads["d_final_state"], grads["dq"], grads["dk"], grads["dv"],
        grads["dlog_alpha"], grads["dbeta"], grads["d_initial_state"], a["batch"], a["seq_len"],
        a["num_heads"], a["head_dim_k"], a["head_dim_v"], a["num_seqs"], a["dtype"], workspace,
        workspace_bytes, a["stream"])


def test_bwd_valid_call_reaches_the_device_check():
    assert call_bwd() in (DEVICE, OK)
    assert call_bwd(initial_state=None, d_final_state=None, d_initial_state=None) in (DEVICE, OK)
    assert call_bwd(dtype=F32) in (DEVICE, OK)  # fp32 at d = 128 is supported here


@pytest.mark.parametrize("name", ["d_out", "dq", "dk", "dv", "dlog_alpha", "dbeta"])
def test_bwd_null_required(name):
    assert call_bwd(**{name: None}) == NULL


def test_bwd_checks():
    a = chunk_args()
    assert call_bwd(workspace=None) == NULL
    assert call_bwd(workspace_bytes=1024) == SHAPE
    assert call_bwd(workspace_bytes=-1) == SHAPE
    assert call_bwd(workspace=(1 << 52) + 8) == ALIGN
    assert call_bwd(dbeta=(1 << 51) + 4) in (DEVICE, OK)  # 4-byte alignment suffices
    assert call_bwd(dq=(1 << 51) + 4) == ALIGN
    assert call_bwd(head_dim_k=96, head_dim_v=96) == UNSUP
    assert call_bwd(head_dim_v=64) == UNSUP
    assert call_bwd(batch=-1) == SHAPE
    assert call_bwd(dq=a["q"]) == ALIAS
    assert call_bwd(workspace=a["k"]) == ALIAS
    same = (1 << 49)
    assert call_bwd(dq=same, dk=same) == ALIAS
    assert call_bwd(batch=0, workspace=None) == OK
    assert call_bwd(num_heads=0, workspace=None) == OK


# ---------------------------------------------------------------- decode_step
def decode_args(**kw):
    b = Buf()
    args = dict(q=b(), k=b(), v=b(), log_alpha=b(), beta=b(), state=b(), out=b(), batch=4,
                num_heads=3, head_dim_k=128, head_dim_v=128, dtype=BF16, stream=None)
    args.update(kw)
    return args


def call_decode(**kw):
    a = decode_args(**kw)
    return _lib.lib().kda_decode_step(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"],
                                      a["state"], a["out"], a["batch"], a["num_heads"],
                                      a["head_dim_k"], a["head_dim_v"], a["dtype"], a["stream"])


@pytest.mark.parametrize("name", ["q", "k", "v", "log_alpha", "beta", "state", "out"])
def test_decode_null(name):
    assert call_decode(**{name: None}) == NULL


@pytest.mark.parametrize("kw", [dict(batch=-1), dict(num_heads=-2), dict(head_dim_k=0)])
def test_decode_bad_sizes(kw):
    assert call_decode(**kw) == SHAPE


@pytest.mark.parametrize("kw", [dict(head_dim_k=128, head_dim_v=64), dict(head_dim_k=32,
                                head_dim_v=32), dict(dtype=3)])
def test_decode_unsupported(kw):
    assert call_decode(**kw) == UNSUP


@pytest.mark.parametrize("name", ["q", "k", "v", "log_alpha", "beta", "state", "out"])
def test_decode_misaligned(name):
    a = decode_args()
    assert call_decode(**{name: a[name] + 2}) == ALIGN


def test_decode_beta_needs_four_bytes_only():
    a = decode_args()
    assert call_decode(beta=a["beta"] + 12) in (DEVICE, OK)


def test_decode_aliasing():
    a = decode_args()
    assert call_decode(out=a["state"] + 64) == ALIAS
    assert call_decode(out=a["q"]) == ALIAS
    assert call_decode(state=a["k"]) == ALIAS


def test_decode_empty_is_ok():
    assert call_decode(batch=0) == OK
    assert call_decode(num_heads=0, q=None, k=None) == OK


def test_decode_valid_arguments_reach_device_check():
    assert call_decode(dtype=F32, head_dim_k=64, head_dim_v=64) in (DEVICE, OK)


# ---------------------------------------------------------------- scalar-gate variants
def call_chunk_sg(**kw):
    a = chunk_args(**kw)
    return _lib.lib().kda_chunk_fwd_scalar_gate(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"],
        a["cu_seqlens"], a["out"], a["final_state"], a["batch"], a["seq_len"],
        a["num_heads"], a["head_dim_k"], a["head_dim_v"], a["num_seqs"], a["dtype"],
        a["stream"])


def test_chunk_scalar_gate_checks():
    a = chunk_args()
    assert call_chunk_sg() in (DEVICE, OK)
    assert call_chunk_sg(log_alpha=None) == NULL
    assert call_chunk_sg(dtype=F32) in (DEVICE, OK)
    assert call_chunk_sg(head_dim_k=96, head_dim_v=96) == UNSUP
    # one float per (token, head): 4-byte alignment suffices
    assert call_chunk_sg(log_alpha=a["log_alpha"] + 4) in (DEVICE, OK)
    assert call_chunk_sg(log_alpha=a["log_alpha"] + 2) == ALIGN
    # the gate array is [B, T, H] floats: an output 2*100*3*4 bytes past it is clear
    assert call_chunk_sg(out=a["log_alpha"] + 2400) in (DEVICE, OK)
    assert call_chunk_sg(out=a["log_alpha"] + 2384) == ALIAS


def call_decode_sg(**kw):
    a = decode_args(**kw)
    return _lib.lib().kda_decode_step_scalar_gate(
        a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["state"], a["out"], a["batch"],
        a["num_heads"], a["head_dim_k"], a["head_dim_v"], a["dtype"], a["stream"])


def test_decode_scalar_gate_checks():
    a = decode_args()
    assert call_decode_sg() in (DEVICE, OK)
    assert call_decode_sg(log_alpha=None) == NULL
    assert call_decode_sg(log_alpha=a["log_alpha"] + 4) in (DEVICE, OK)
    assert call_decode_sg(log_alpha=a["log_alpha"] + 1) == ALIGN
    # [B, H] = 4 * 3 floats = 48 bytes
    assert call_decode_sg(out=a["log_alpha"] + 48) in (DEVICE, OK)
    assert call_decode_sg(out=a["log_alpha"] + 32) == ALIAS


def test_debug_mode_keeps_host_validation(monkeypatch):
    """KDA_DEBUG adds device-side checks after validation; the host checks
    and their codes are unchanged, and without a GPU a valid call still stops
    at the device check."""
    monkeypatch.setenv("KDA_DEBUG", "1")
    assert call_chunk(q=None) == NULL
    assert call_chunk(head_dim_k=96, head_dim_v=96) == UNSUP
    assert call_chunk() in (DEVICE, OK)
    assert call_seg(workspace=None) == NULL
