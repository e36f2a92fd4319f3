"""CPU checks of the comparators' allowances (test infrastructure)."""
import numpy as np
import pytest

from checks import check_f32, fp8_window_bound


def test_window_bound_covers_the_dropped_products():
    # one group: 2^8 and seven products of 2^-6, 14 binades below it; the FP8
    # MFMA returns 2^8, so the allowance must reach the 7 * 2^-6 it drops
    p = np.array([[2.0 ** 8] + [2.0 ** -6] * 7])
    assert fp8_window_bound(p)[0] >= 7 * 2.0 ** -6
    # products within 6 binades of the group maximum need nothing
    assert fp8_window_bound(np.array([[2.0 ** 4] + [2.0 ** -2] * 7]))[0] == 0.0


def test_window_bound_group_scale_and_groups():
    p = np.array([[1.0] + [2.0 ** -20] * 7 + [4.0] + [2.0 ** -18] * 7])
    b = fp8_window_bound(p)
    g = fp8_window_bound(p, gscale=np.array([[3.0, 0.5]]))
    # each group: 7 products below its window bit, taken whole; twice the sum
    assert b[0] == pytest.approx(2 * (7 * 2.0 ** -20 + 7 * 2.0 ** -18))
    assert g[0] == pytest.approx(2 * (3.0 * 7 * 2.0 ** -20 + 0.5 * 7 * 2.0 ** -18))


def test_check_f32_extra_allowance():
    c64, b = np.array([1.0]), np.array([1.0])
    with pytest.raises(AssertionError):
        check_f32(np.array([1.0 + 2e-5]), c64, b)
    check_f32(np.array([1.0 + 2e-5]), c64, b, extra=np.array([1.5e-5]))
