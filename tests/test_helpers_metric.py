"""The parity metrics themselves (CPU): what each one flags."""

import numpy as np

from tests.helpers import HEAD_FLOOR, block_rel_err, head_rel_err


def test_head_metric_sees_errors_in_small_heads():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 4, 16))
    ref[:, :, 8:] *= 1e-2                       # head 1 is small next to head 0
    got = ref.copy()
    got[1, 2, 9] += 1e-5                        # an error of 1e-5 in the small head
    assert block_rel_err(got, ref, 1) < 1e-4    # hidden by the block's scale
    assert head_rel_err(got, ref, 1, 2) > 1e-4  # seen against the head's own scale
    assert head_rel_err(ref, ref, 1, 2) == 0.0


def test_head_metric_floor_and_exact_zeros():
    ref = np.zeros((2, 1, 4))
    ref[0, 0, :2] = 1.0                         # head 1 of atom 0 is exactly zero
    got = ref.copy()
    got[0, 0, 3] = 1e-6                         # tiny noise where the reference is 0
    assert np.isclose(head_rel_err(got, ref, 0, 2), 1e-6 / HEAD_FLOOR)
    assert head_rel_err(ref, ref, 0, 2) == 0.0  # 0/0 counts as 0
    got[1, 0, 0] = 1.0                          # an all-zero block answered non-zero
    assert head_rel_err(got, ref, 0, 2) == np.inf
    got[0, 0, 0] = np.nan
    assert head_rel_err(got, ref, 0, 2) == np.inf
