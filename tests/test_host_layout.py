"""Host-side checks of the backward's workspace slot layout (no GPU).

kda_chunk_bwd keeps one state per 16-token chunk and head in each workspace
region: chunk j of sequence n, which starts at token t0, uses slot
t0 // 16 + n + j, and a region has total_tokens // 16 + num_seqs + 1 slots.
The gradient kernel runs one workgroup per slot and finds its sequence as the
last n whose first slot is at or before the slot.  These tests check, for
random packings (empty sequences included), that the slot ranges of the
sequences are disjoint, increasing and inside the region, and that this
search maps every used slot back to its own sequence and chunk.
"""
import numpy as np
import pytest

import gated_delta_rule_81_amd._lib as _lib

CHUNK = 16


def slot_ranges(lengths):
    starts = np.concatenate([[0], np.cumsum(lengths)])
    return [(int(starts[n]) // CHUNK + n, int(starts[n]) // CHUNK + n + -(-int(L) // CHUNK))
            for n, L in enumerate(lengths)], starts


def sequence_of_slot(slot, starts):
    """The kernel's bisection: the last n with starts[n] // 16 + n <= slot."""
    lo, hi = 0, len(starts) - 2
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if int(starts[mid]) // CHUNK + mid <= slot:
            lo = mid
        else:
            hi = mid - 1
    return lo


@pytest.mark.parametrize("seed", range(20))
def test_slot_ranges_disjoint_and_inside(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    lengths = rng.integers(0, 200, size=n)
    lengths[rng.random(n) < 0.2] = 0  # empty sequences
    ranges, starts = slot_ranges(lengths)
    total = int(starts[-1])
    region = total // CHUNK + n + 1
    prev_end = 0
    for (a, b), L in zip(ranges, lengths):
        assert b - a == -(-int(L) // CHUNK)
        assert a >= prev_end  # disjoint and increasing
        assert b <= region
        prev_end = max(prev_end, b)
    # every used slot maps back to its own sequence and chunk (a range ends at
    # or before the next sequence's first slot, so the search stops at m)
    for m, (a, b) in enumerate(ranges):
        for c, slot in enumerate(range(a, b)):
            k = sequence_of_slot(slot, starts)
            assert k == m
            assert slot - (int(starts[k]) // CHUNK + k) == c
    # slots used by no sequence are recognised as such (chunk index out of range)
    used = {s for a, b in ranges for s in range(a, b)}
    for slot in range(region):
        k = sequence_of_slot(slot, starts)
        c = slot - (int(starts[k]) // CHUNK + k)
        inside = 0 <= c < -(-int(lengths[k]) // CHUNK)
        assert inside == (slot in used)


def test_workspace_size_holds_two_regions():
    f = _lib.lib().kda_chunk_bwd_workspace_size
    for total, n, h, d in [(32768, 1, 96, 128), (4096, 1, 32, 128), (333, 7, 3, 64)]:
        region = (total // CHUNK + n + 1) * h * d * d * 4
        assert f(total, n, h, d) == 2 * region + 16 * n * h * 4  # + flag words
