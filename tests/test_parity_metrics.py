"""The parity metrics of gpu_util on hand-made arrays (no GPU)."""
import numpy as np

from gpu_util import local_errors, unit_rel_errors


def test_metrics_localise_an_error_in_small_outputs():
    rng = np.random.default_rng(0)
    B, T, H, d = 1, 300, 2, 8
    ref = rng.standard_normal((B, T, H, d))
    ref[0, :64] *= 1e-3            # an early window of small outputs
    o = ref.copy()
    o[0, 10, 1, 3] += 2e-4         # ~5 % of that window's scale, ~5e-5 of the unit's
    slices = [(0, 0, T)]
    eo, _, unit = unit_rel_errors(o, None, ref, None, slices, H)
    ew, ee = local_errors(o, ref, slices, H)
    assert eo < 1e-4 and unit == (0, 1)          # hidden by the unit's largest value
    assert ew > 2e-2                             # the window sees it
    assert ee > 1e-2
    ew0, ee0 = local_errors(ref, ref, slices, H)
    assert ew0 == 0.0 and ee0 == 0.0


def test_windows_cover_a_ragged_tail_and_packed_units():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((1, 130, 1, 4))
    o = ref.copy()
    o[0, 129, 0, 0] += 1.0         # last token of the second sequence (a 2-token tail window)
    ew, _ = local_errors(o, ref, [(0, 0, 60), (0, 60, 130)], 1)
    assert ew > 0.1
    z = np.zeros((1, 10, 1, 4))
    bad = z.copy()
    bad[0, 3, 0, 1] = 1e-9         # any error where the reference window is all zero
    assert local_errors(bad, z, [(0, 0, 10)], 1)[0] == float("inf")
