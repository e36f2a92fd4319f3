"""CPU checks of the comparators' allowances (test infrastructure)."""
import numpy as np
import pytest

from checks import check_f32, e4m3_window_exponent, fp8_window_bound


def test_window_exponent():
    v = np.array([448.0, 1.0, 1.875, 2.0 ** -6, 2.0 ** -7, 2.0 ** -9, 0.0, -3.0])
    assert e4m3_window_exponent(v).tolist() == [8, 0, 0, -6, -6, -6, -6, 1]


def test_window_bound_dropped_and_kept():
    # 2^8 * 2^-6 sets the exponent sum 2: the window's last bit is 2^-11 and
    # the seven 2^-12 products are lost whole
    a = np.array([2.0 ** 8] + [2.0 ** -6] * 7)
    w = np.full(8, 2.0 ** -6)
    assert fp8_window_bound(a, w) == 7 * 2.0 ** -12
    # 16 * 2^-6 (exponent sum -2): 2^-9 * 2^-6 = 2^-15 is the last bit, kept
    a = np.array([16.0] + [2.0 ** -9] * 7)
    assert fp8_window_bound(a, w) == 0.0
    # one binade more and it is lost
    a = np.array([32.0] + [2.0 ** -9] * 7)
    assert fp8_window_bound(a, w) == 7 * 2.0 ** -15


def test_window_bound_partial_truncation():
    # 1.875 * 2^-10 against the last bit 2^-11 loses 0.75 * 2^-11 (truncation
    # toward zero keeps 1.5 * 2^-10), whatever the signs
    a = np.array([256.0, 1.875 * 2.0 ** -4] + [0.0] * 6)
    w = np.full(8, 2.0 ** -6)
    assert fp8_window_bound(a, w) == 0.75 * 2.0 ** -11
    assert fp8_window_bound(-a, w) == 0.75 * 2.0 ** -11
    assert fp8_window_bound(a * np.array([-1, 1, 1, 1, 1, 1, 1, 1]), w) == 0.75 * 2.0 ** -11


def test_window_bound_follows_exponent_sums():
    # 448 * 6 * 2^-6 = 42 has value exponent 5 but exponent sum 4: the last
    # bit is 2^-9, so seven products of exactly 2^-9 are kept
    a = np.array([448.0] + [2.0 ** -3] * 7)
    w = np.array([6.0] + [1.0] * 7) * 2.0 ** -6
    assert fp8_window_bound(a, w) == 0.0


def test_window_bound_groups_and_scales():
    a = np.concatenate([[2.0 ** 8], np.full(7, 2.0 ** -6), [2.0 ** 4], np.full(7, 2.0 ** -9)])
    w = np.full(16, 2.0 ** -6)
    # group 0 loses 7 * 2^-12, group 1 (exponent sum -2, last bit 2^-15) nothing
    assert fp8_window_bound(a, w) == 7 * 2.0 ** -12
    assert fp8_window_bound(a, w, gscale=np.array([3.0, 0.5])) == 3 * 7 * 2.0 ** -12
    # a product with a zero operand does not place the window: a zero next to
    # 448 leaves the one real product exact; an all-zero group loses nothing
    a = np.array([0.0, 2.0 ** -9] + [0.0] * 6)
    w = np.array([448.0, 2.0 ** -9] + [0.0] * 6)
    assert fp8_window_bound(a, w) == 0.0
    assert fp8_window_bound(np.zeros(8), np.full(8, 448.0)) == 0.0
    # leading dimensions
    assert fp8_window_bound(np.stack([a, a]), w).shape == (2,)


def test_check_f32_extra_allowance():
    c64, b = np.array([1.0]), np.array([1.0])
    with pytest.raises(AssertionError):
        check_f32(np.array([1.0 + 2e-5]), c64, b)
    check_f32(np.array([1.0 + 2e-5]), c64, b, extra=np.array([1.5e-5]))
