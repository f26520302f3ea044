"""Pins for the oracle's power-of-two scale option (CPU only).

The scale rule (reading Q13 of the oracle): S is the smallest power of two with 448 * S >= amax,
at least 2^-127, and 1 for an all-zero group. Independent references: a group worked by hand
(golden fixture), exact rational checks of minimality on random and extreme amax values, closed
forms, and agreement with the FP32-scale quantizer wherever amax / 448 is itself a power of two.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant
from tests.exact import f32_to_fraction
from tests.test_oracle_quant import bf16_bits, random_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_group_pow2():
    d = json.load(open(os.path.join(GOLDEN, "worked_group_pow2.json")))
    x = np.zeros(128, dtype=np.float32)
    want = np.zeros(128, dtype=np.uint8)
    for e in d["entries"]:
        x[e["idx"]] = np.float32(float(e["x"]))
        want[e["idx"]] = int(e["code"], 16)
    bits = bf16_bits(x)
    q, sa = quant.quant_act_tok128(bits[None, :], scale="pow2")
    assert sa[0, 0] == np.float32(d["scale"])
    assert np.array_equal(q[0], want)
    w = np.zeros((256, 128), dtype=np.uint16)
    w[130] = bits
    wq, sw = quant.quant_weight_blk128(w, scale="pow2")
    assert sw[1, 0] == np.float32(d["scale"]) and sw[0, 0] == np.float32(1.0)
    assert np.array_equal(wq[130], want)


@pytest.mark.parametrize("amax,S", [(0.0, 1.0), (3.5, 2.0 ** -7), (3.75, 2.0 ** -6), (448.0, 1.0),
                                    (449.0, 2.0), (1.0, 2.0 ** -8), (896.0, 2.0), (897.0, 4.0),
                                    (0.875 * 2.0 ** -118, 2.0 ** -127),
                                    (2.0 ** -130, 2.0 ** -127), (3.3895313892515355e38, 2.0 ** 120)])
def test_closed_forms(amax, S):
    assert quant.scale_from_amax_pow2(np.float32(amax)) == np.float32(S)


def _check_minimal(amax32):
    S = quant.scale_from_amax_pow2(amax32)
    for a, s in zip(amax32.ravel(), S.ravel()):
        fa, fs = f32_to_fraction(a), f32_to_fraction(s)
        if fa == 0:
            assert fs == 1
            continue
        m, e = np.frexp(np.float64(s))
        assert m == 0.5, "S must be a power of two"
        assert 448 * fs >= fa                          # no quotient leaves +-448
        assert fs == Fraction(2) ** -127 or 448 * fs / 2 < fa  # and no smaller power would do


def test_minimal_power_of_two_random_and_extremes():
    rng = np.random.default_rng(7)
    a = np.abs(rng.standard_normal(20000)).astype(np.float32) * np.float32(2.0) ** rng.integers(
        -140, 120, 20000).astype(np.float32)
    a = a[np.isfinite(a)]
    bf = (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # bf16-representable amax
    edge = np.array([448 * 2.0 ** k for k in range(-127, 118)] + [np.nextafter(np.float32(448 * 2.0 ** k),
                    np.float32(np.inf)) for k in range(-120, 110)], dtype=np.float32)
    _check_minimal(np.concatenate([bf, edge, np.float32([0.0])]))


def test_quotients_stay_in_range_and_amax_lands_high():
    for seed in range(5):
        w = random_bf16((256, 384), seed=40 + seed, scale=10.0 ** (seed - 2))
        q, s = quant.quant_weight_blk128(w, scale="pow2")
        v = np.abs(e4m3.decode(q).astype(np.float64))
        assert np.nanmax(v) <= 448 and not np.any(np.isnan(v))
        x = quant.bf16_bits_to_f32(w).astype(np.float64)
        for i in range(2):
            for j in range(3):
                blk = np.abs(x[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
                r = blk.max() / float(s[i, j])
                assert 224 < r <= 448  # the amax element lands in the top binade


def test_agrees_with_fp32_scales_when_amax_over_448_is_a_power_of_two():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * 0.5).astype(np.float32)
    x = np.clip(x, -1.75, 1.75)
    x[:, 0] = 1.75   # amax of every group = 1.75 = 448 * 2^-8
    x[:, 128] = -1.75
    bits = bf16_bits((x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32))
    q32, s32 = quant.quant_act_tok128(bits, scale="fp32")
    q2, s2 = quant.quant_act_tok128(bits, scale="pow2")
    assert np.all(s32 == np.float32(2.0 ** -8)) and np.array_equal(s32, s2)
    assert np.array_equal(q32, q2)


def test_pow2_differs_from_fp32_elsewhere():
    w = random_bf16((128, 128), seed=11)
    _, s32 = quant.quant_weight_blk128(w)
    _, s2 = quant.quant_weight_blk128(w, scale="pow2")
    assert s2[0, 0] >= s32[0, 0] and s2[0, 0] < 2 * s32[0, 0]


def test_unknown_scale_rejected():
    with pytest.raises(ValueError):
        quant.quant_act_tok128(np.zeros((1, 128), np.uint16), scale="e8m0")
