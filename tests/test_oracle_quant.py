"""Pins of oracle.quant: hand-worked scale/code examples, the half-scale rounding
bound, the code range, and the packed bit positions."""
import json
import os

import numpy as np
import pytest

from oracle import quant
from oracle.numerics import bf16_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_scale_and_codes_hand_worked():
    with open(os.path.join(GOLDEN, "quant_hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        r = np.array([case["residual"]], np.float32)
        d = r.shape[1]
        lay = quant.channel_layout(d, case["bits"], d)
        q, s = quant.quantize_groups(r, lay)
        assert s[0, 0] == np.float32(case["scale"]), case["name"]
        assert q[0].tolist() == case["codes"], case["name"]


def test_scale_formula_closed_form():
    amax = np.array([3.0, 1.0, 0.0, 100.5], np.float32)
    # b = 2: 2^(b-1) - 1 = 1 -> the scale is amax itself, rounded to bf16
    assert quant.scale_of(amax, 2).tolist() == bf16_rne(amax).tolist()
    # b = 4: divisor 7
    assert quant.scale_of(np.float32(7.0), 4) == np.float32(1.0)


@pytest.mark.parametrize("bits", [2, 4])
def test_half_scale_bound_and_range(bits):
    rng = np.random.default_rng(bits)
    r = (rng.standard_normal((2000, 128)) * rng.uniform(0.01, 100, (2000, 1))).astype(np.float32)
    r[::7, 3] *= 1000.0                      # outliers
    r[5, :] = 0.0                            # an all-zero token (S = 0)
    lay = quant.channel_layout(128, bits, 32)
    q, s = quant.quantize_groups(r, lay)
    srow = quant.expand_scales(s, lay)
    err = np.abs(r.astype(np.float64) - srow.astype(np.float64) * q)
    # |r - S q| <= S / 2, up to the float32 rounding of r / S
    assert np.all(err <= srow.astype(np.float64) * (0.5 + 2.0 ** -20))
    qmax = 2 ** (bits - 1) - 1
    assert q.min() >= -qmax and q.max() <= qmax   # the clamp never binds
    assert np.all(q[5] == 0) and np.all(s[5] == 0)


def test_layout_uniform_and_mixed():
    lay = quant.channel_layout(128, 2, 32)
    assert lay.words == 8 and len(lay.groups) == 4
    lay4 = quant.channel_layout(128, 4, 32)
    assert lay4.words == 16
    perm = np.concatenate([np.arange(100, 126), np.arange(0, 100), np.arange(126, 128)])
    mix = quant.channel_layout(128, 2, 32, n_int4=26, perm=perm)
    # 26 x 4 bits -> 4 words (padded), 102 x 2 bits -> 7 words
    assert mix.class_word0 == (0, 4) and mix.words == 11
    assert [len(g.channels) for g in mix.groups] == [26, 32, 32, 32, 6]
    assert [g.bits for g in mix.groups] == [4, 2, 2, 2, 2]


def test_single_code_bit_placement():
    lay = quant.channel_layout(128, 2, 32)
    for ch in [0, 1, 15, 16, 31, 127]:
        q = np.full((1, 128), -1, np.int8)   # u = 1 everywhere
        q[0, ch] = 1                           # u = 3 at ch
        w = quant.pack_codes(q, lay)
        for wi in range(8):
            expect = 0x55555555                # 01 in every 2-bit slot
            if wi == ch // 16:
                expect |= 3 << (2 * (ch % 16))
            assert int(w[0, wi]) == expect
    lay4 = quant.channel_layout(128, 4, 32)
    q = np.zeros((1, 128), np.int8)            # u = 8 everywhere
    q[0, 13] = -8 + 15                         # u = 15
    w = quant.pack_codes(q, lay4)
    assert int(w[0, 1]) == (0x88888888 & ~(0xF << 20)) | (0xF << 20)


def test_pack_roundtrip_mixed():
    rng = np.random.default_rng(5)
    perm = rng.permutation(128)
    mix = quant.channel_layout(128, 2, 32, n_int4=26, perm=perm)
    q = np.zeros((50, 128), np.int8)
    for ch in range(128):
        b = int(mix.ch_bits[ch])
        q[:, ch] = rng.integers(-(2 ** (b - 1)), 2 ** (b - 1), 50)
    assert np.array_equal(quant.unpack_codes(quant.pack_codes(q, mix), mix), q)
