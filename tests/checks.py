"""Comparators shared by the parity tests (test infrastructure).

Tolerances, as the workload fixes them:
  * FP32 accumulators: |C32 - C64| <= 1e-5 * B, where B = sum_k |a_k * w_k|
    (the same scale factors applied); where B == 0 the result must be 0.
  * BF16 outputs: within one BF16 ulp of the oracle value rounded to nearest
    even directly from FP64 (ordinal distance of the bit patterns, +-0 equal).
Both refuse empty inputs and NaN, so a vacuous comparison cannot pass.
"""
import numpy as np

REL_TOL = 1e-5


def check_f32(c32, c64, bound, rel=REL_TOL, what="", extra=None):
    """extra: an additional absolute allowance per output (the FP8 MFMA
    summation window, fp8_window_bound), added to rel * bound."""
    c32 = np.asarray(c32, dtype=np.float64).ravel()
    c64 = np.asarray(c64, dtype=np.float64).ravel()
    bound = np.asarray(bound, dtype=np.float64).ravel()
    assert c32.size > 0 and c32.size == c64.size == bound.size, f"{what}: empty or mismatched"
    assert rel > 0, "degenerate tolerance"
    assert np.all(np.isfinite(c32)), f"{what}: non-finite GPU values"
    assert np.all(np.isfinite(c64)) and np.all(np.isfinite(bound)), f"{what}: non-finite oracle"
    err = np.abs(c32 - c64)
    lim = rel * bound
    if extra is not None:
        extra = np.asarray(extra, dtype=np.float64).ravel()
        assert extra.size == c32.size and np.all(extra >= 0), f"{what}: bad allowance"
        lim = lim + extra
    bad = np.where((bound == 0) & (c32 != 0) | (err > lim))[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {c32.size} outside 1e-5*B; first at {bad[:5]}: "
                           f"gpu {c32[bad[:5]]} oracle {c64[bad[:5]]} B {bound[bad[:5]]}")
    nz = bound > 0
    return float(np.max(err[nz] / bound[nz])) if nz.any() else 0.0


def bf16_ordinal(bits):
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_bf16(bits, ref_bits, what=""):
    bits = np.asarray(bits).ravel()
    ref_bits = np.asarray(ref_bits).ravel()
    assert bits.size > 0 and bits.size == ref_bits.size, f"{what}: empty or mismatched"
    nan = (bits.astype(np.int64) & 0x7FFF) > 0x7F80
    assert not nan.any(), f"{what}: NaN in GPU output"
    d = np.abs(bf16_ordinal(bits) - bf16_ordinal(ref_bits))
    bad = np.where(d > 1)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {bits.size} beyond 1 BF16 ulp; first at "
                           f"{bad[:5]}: gpu {bits[bad[:5]]} oracle {ref_bits[bad[:5]]}")
    return int(d.max())


def fp8_window_bound(p, gscale=None):
    """Extra error allowance for sums formed by gfx950's FP8 MFMAs.

    Measured on the device (one large product plus several tiny ones in one
    instruction): the FP8 and MX-FP8 MFMAs sum each aligned group of 8
    products of one lane in a fixed-point window whose lowest kept bit is 13
    binades below the group's largest product; bits below it are dropped (a
    product below the window is lost), while group sums are added in FP32.
    A product with 8 significant bits loses nothing when it lies within 6
    binades of the group maximum.  Per group the error is thus below
    sum over k of min(|p_k|, 2^(e-13)) for the products with |p_k| < 2^(e-6),
    e = floor(log2(max |p|)).  Returns twice that sum over all groups.
    p: products [..., K] (FP64, K % 8 == 0, groups aligned to 8) as the MFMA
    forms them.  gscale: optional factor per group of 8 ([..., K/8]) that is
    applied to a group's sum after the MFMA (a block scale that is not a power
    of two), multiplied into that group's bound."""
    a = np.abs(np.asarray(p, dtype=np.float64))
    a = a.reshape(a.shape[:-1] + (a.shape[-1] // 8, 8))
    mx = a.max(axis=-1, keepdims=True)
    e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    q = 2.0 ** (e - 13)
    small = a < 2.0 ** (e - 6)
    g = (np.minimum(a, q) * small).sum(axis=-1)
    if gscale is not None:
        g = g * np.abs(np.asarray(gscale, dtype=np.float64))
    return 2.0 * g.sum(axis=-1)
