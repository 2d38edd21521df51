"""CPU tests of the parity metrics the GPU tests use (tests/parity.py): the
slice metric agrees with the plain per-slice definition, and the row metric
catches one wrong row that the slice metric cannot see."""
import numpy as np

from parity import ROW_TOL, TOL, max_rel_l2, slice_row_errors, state_errors

import torch


def _case(T=4096, h=3, d=128, seed=0):
    rng = np.random.default_rng(seed)
    ref = rng.normal(size=(T, h, d))
    got = ref * (1 + 4e-3 * rng.normal(size=ref.shape))
    return got, ref


def test_slice_metric_matches_definition():
    got, ref = _case()
    starts = [0, 0, 1000, 1001, 4096]  # an empty and a one-token sequence
    slice_err, _ = slice_row_errors(got, ref, starts)
    pairs = [(got[a:b, j], ref[a:b, j]) for a, b in zip(starts[:-1], starts[1:]) if b > a
             for j in range(ref.shape[1])]
    assert np.isclose(slice_err, max_rel_l2(pairs), rtol=1e-9)


def test_one_wrong_row_fails_rows_not_slices():
    got, ref = _case(T=32768, h=2)
    starts = [0, 32768]
    s0, r0 = slice_row_errors(got, ref, starts)
    assert s0 < TOL[torch.bfloat16] and r0 < ROW_TOL[torch.bfloat16]
    bad = got.copy()
    bad[12345, 1] = 0.0  # one token row lost
    s1, r1 = slice_row_errors(bad, ref, starts)
    assert s1 < TOL[torch.bfloat16]  # the slice metric cannot see it ...
    assert r1 > 0.9  # ... the row metric does
    bad = got.copy()
    bad[777, 0] = ref[778, 0]  # another token's row
    assert slice_row_errors(bad, ref, starts)[1] > 0.5


def test_small_rows_judged_against_the_slice_scale():
    """A row whose reference is near zero is judged relative to the slice's
    typical row, not to its own tiny norm."""
    _, ref = _case(T=64, h=1)
    ref[5] *= 1e-6
    got = ref.copy()
    got[5] = ref[5] + 1e-5  # an absolute error far below the slice's row scale
    err = slice_row_errors(got, ref, [0, 64])[1]
    assert 0 < err < 1e-3
    # relative to its own norm the same row would be off by a factor ~100
    assert np.linalg.norm(got[5] - ref[5]) / np.linalg.norm(ref[5]) > 10


def test_state_rows():
    rng = np.random.default_rng(1)
    ref = rng.normal(size=(2, 3, 64, 64))
    got = ref.copy()
    s, r = state_errors(got, ref)
    assert s == 0 and r == 0
    got[1, 2, 17] = -ref[1, 2, 17]  # one value row flipped
    s, r = state_errors(got, ref)
    assert np.isclose(s, 2 / 8, rtol=0.2) and r > 1.5
