"""Pins of oracle.numerics against hand-worked bit patterns and exact rationals."""
from fractions import Fraction

import numpy as np

from oracle.numerics import bf16_rne, bf16_bits, bf16_from_bits, group_sums_exact


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def test_bf16_rne_hand_worked():
    # (float32 bit pattern, expected bf16 pattern); the low 16 bits decide:
    # below 0x8000 -> down, above -> up, exactly 0x8000 -> to the even upper half.
    cases = [
        (0x3F800000, 0x3F80),   # 1.0 exact
        (0x3F808000, 0x3F80),   # 1 + 2^-8: tie, 0x3F80 is even -> stays
        (0x3F818000, 0x3F82),   # 1 + 3*2^-8: tie, 0x3F81 is odd -> up to even
        (0x3F808001, 0x3F81),   # just above the tie -> up
        (0x3F807FFF, 0x3F80),   # just below the tie -> down
        (0xBF818000, 0xBF82),   # negative tie, magnitude rounds to even
        (0x3EDB6DB7, 0x3EDB),   # fp32(3/7): low half 0x6DB7 < 0x8000 -> down
        (0x7F7F8000, 0x7F80),   # rounds up into the next binade (infinity pattern)
        (0x00000000, 0x0000),
    ]
    for src, want in cases[:-2] + cases[-1:]:
        got = bf16_bits(bf16_rne(_f32(src)))
        assert int(got) == want, (hex(src), hex(int(got)), hex(want))


def test_bf16_values_are_fixed_points():
    rng = np.random.default_rng(0)
    pats = rng.integers(0, 1 << 16, 20000).astype(np.uint16)
    vals = bf16_from_bits(pats)
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(bf16_rne(vals).view(np.uint32), vals.view(np.uint32))


def test_bf16_rne_is_nearest():
    # brute force: the result is one of the two bf16 neighbours and the closer one
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 6, 5000)).astype(np.float32)
    r = bf16_rne(x)
    u = x.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32)
    hi = ((u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32)
    for xi, ri, a, b in zip(x.astype(np.float64), r.astype(np.float64), lo.astype(np.float64), hi.astype(np.float64)):
        assert ri in (a, b)
        assert abs(ri - xi) <= min(abs(a - xi), abs(b - xi))


def test_group_sums_exact_against_rationals():
    rng = np.random.default_rng(2)
    n, d, c = 300, 5, 7
    # wide dynamic range (forces the correctly-rounded fallback on some entries)
    y = (rng.standard_normal((n, d)) * 10.0 ** rng.integers(-12, 4, (n, d))).astype(np.float32)
    labels = rng.integers(0, c, n)
    labels[labels == 6] = 5          # leave group 6 empty
    s = group_sums_exact(y, labels, c)
    for j in range(c):
        for k in range(d):
            exact = sum((Fraction(float(v)) for v in y[labels == j, k]), Fraction(0))
            assert s[j, k] == float(exact), (j, k)
    assert np.all(s[6] == 0)
