"""Host check of the index arithmetic the kernels' epilogues rely on.

The QKV epilogue splits a column into (head, pair within the head, group)
with floor(x / d) computed as trunc((x + 1/2) * inv), inv the hardware
reciprocal of d (within one ulp of 1/d), instead of a software integer
division.  The claim behind it: for 0 <= x < 2^21 the truncation is exact,
because (x + 1/2)/d lies at least 1/(2d) away from an integer while the
reciprocal's error and the product's rounding move it by less than that.
This test replays those fp32 steps with numpy over every x the epilogue can
see at these sizes, for every divisor up to 2048 and for the reciprocal
rounded to nearest or one ulp off either way."""
import numpy as np


def _div_small(x, inv):
    xf = x.astype(np.float32) + np.float32(0.5)
    return (xf * np.float32(inv)).astype(np.int64)  # fp32 product, truncation toward zero


def test_div_small_exact_over_index_ranges():
    x = np.arange(0, 1 << 16, dtype=np.int64)  # column, pair and head indices stay far below this
    for d in range(1, 2049):
        ref = x // d
        inv = np.float32(1.0) / np.float32(d)
        for r in (inv, np.nextafter(inv, np.float32(0)), np.nextafter(inv, np.float32(1))):
            got = _div_small(x, r)
            assert np.array_equal(got, ref), (d, r, int(np.flatnonzero(got != ref)[0]))


def test_div_small_exact_at_the_stated_bound():
    # the largest x of the claim, against divisors whose multiples sit just below it
    top = (1 << 21) - 1
    for d in (3, 5, 7, 21, 168, 1000, 2047):
        x = np.array([top, top - 1, (top // d) * d, (top // d) * d - 1], dtype=np.int64)
        inv = np.float32(1.0) / np.float32(d)
        for r in (inv, np.nextafter(inv, np.float32(0)), np.nextafter(inv, np.float32(1))):
            assert np.array_equal(_div_small(x, r), x // d), (d, r)
