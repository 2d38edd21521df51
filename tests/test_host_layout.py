"""Host-side checks of the backward's workspace slot layout (no GPU).

kda_chunk_bwd keeps one state per 16-token chunk and head in each workspace
region: chunk j of sequence n, which starts at token t0, uses slot
t0 // 16 + n + j, and a region has total_tokens // 16 + num_seqs + 1 slots.
The gradient kernel runs one workgroup per slot and finds its sequence as the
last n whose first slot is at or before the slot.

The functions under test are the kernels' own: csrc/kda_slots.h, which the
states, chain, token-level and gradient kernels include, is compiled for the
host (tests/hip/slots_host.cpp) and called through ctypes.  The expectations
are the layout as stated above, written out here: for random packings (empty
sequences included) the slot ranges of the sequences are disjoint, increasing
and inside the region, and every slot maps back to its own sequence and chunk,
or to no chunk at all.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import gated_delta_rule_81_amd._lib as _lib

CHUNK = 16
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_81_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def slots(tmp_path_factory):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    so = str(tmp_path_factory.mktemp("slots") / "libslots_host.so")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-fPIC", "-shared", "-I", CSRC,
           os.path.join(ROOT, "tests", "hip", "slots_host.cpp"), "-o", so]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    lib = ctypes.CDLL(so)
    lib.kda_test_first_slot.restype = ctypes.c_longlong
    lib.kda_test_first_slot.argtypes = [ctypes.c_longlong, ctypes.c_int]
    lib.kda_test_region_slots.restype = ctypes.c_longlong
    lib.kda_test_region_slots.argtypes = [ctypes.c_longlong, ctypes.c_longlong]
    lib.kda_test_slot_sequence.restype = ctypes.c_int
    lib.kda_test_slot_sequence.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_longlong,
                                           ctypes.POINTER(ctypes.c_int)]
    return lib


def owner(lib, cu, num_seqs, seq_len, total, slot):
    """(sequence, chunk) that the kernels' slot_sequence gives for `slot`."""
    chunk = ctypes.c_int(-99)
    ptr = None if cu is None else cu.ctypes.data
    n = lib.kda_test_slot_sequence(ptr, num_seqs, seq_len, total, slot, ctypes.byref(chunk))
    return n, chunk.value


def slot_ranges(lengths):
    starts = np.concatenate([[0], np.cumsum(lengths)])
    return [(int(starts[n]) // CHUNK + n, int(starts[n]) // CHUNK + n + -(-int(L) // CHUNK))
            for n, L in enumerate(lengths)], starts


@pytest.mark.parametrize("seed", range(20))
def test_slot_ranges_disjoint_and_inside(slots, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    lengths = rng.integers(0, 200, size=n)
    lengths[rng.random(n) < 0.2] = 0  # empty sequences
    ranges, starts = slot_ranges(lengths)
    total = int(starts[-1])
    region = total // CHUNK + n + 1
    assert slots.kda_test_region_slots(total, n) == region
    cu = starts.astype(np.int32)
    prev_end = 0
    for m, ((a, b), L) in enumerate(zip(ranges, lengths)):
        assert slots.kda_test_first_slot(int(starts[m]), m) == a
        assert b - a == -(-int(L) // CHUNK)
        assert a >= prev_end  # disjoint and increasing
        assert b <= region
        prev_end = max(prev_end, b)
    # every used slot maps back to its own sequence and chunk
    for m, (a, b) in enumerate(ranges):
        for c, slot in enumerate(range(a, b)):
            assert owner(slots, cu, n, 0, total, slot) == (m, c)
    # slots used by no sequence are recognised as such (chunk index out of range)
    used = {s for a, b in ranges for s in range(a, b)}
    for slot in range(region):
        k, c = owner(slots, cu, n, 0, total, slot)
        assert 0 <= k < n
        inside = 0 <= c < -(-int(lengths[k]) // CHUNK)
        assert inside == (slot in used)


@pytest.mark.parametrize("seq_len,num_seqs", [(16, 1), (33, 3), (4096, 2), (15, 5)])
def test_equal_length_sequences(slots, seq_len, num_seqs):
    """No offsets: sequence m starts at m * seq_len."""
    ranges, _ = slot_ranges([seq_len] * num_seqs)
    total = seq_len * num_seqs
    for m, (a, b) in enumerate(ranges):
        for c, slot in enumerate(range(a, b)):
            assert owner(slots, None, num_seqs, seq_len, total, slot) == (m, c)


def test_offsets_out_of_range_are_clamped(slots):
    """Offsets outside [0, total] (the kernels clamp them) still give a
    sequence in range for every slot, so the bisection ends for any input."""
    total = 100
    cu = np.array([-50, 40, 1000, 60, 100], dtype=np.int32)  # clamped: 0, 40, 100, 60, 100
    n = len(cu) - 1
    for slot in range(total // CHUNK + n + 1):
        k, _ = owner(slots, cu, n, 0, total, slot)
        assert 0 <= k < n


def test_workspace_size_holds_two_regions():
    f = _lib.lib().kda_chunk_bwd_workspace_size
    for total, n, h, d in [(32768, 1, 96, 128), (4096, 1, 32, 128), (333, 7, 3, 64)]:
        region = (total // CHUNK + n + 1) * h * d * d * 4
        assert f(total, n, h, d) == 2 * region + 16 * n * h * 4  # + flag words
