"""Pins for the oracle's E4M3 codec (CPU only).

The independent references are (a) the facts the pages state (4 exponent bits, 3 mantissa bits,
range +-448: FP8-RL write-up, section 1), (b) torch's own float8_e4m3fn type, a separate
implementation of the OCP E4M3 format, and (c) exact rational arithmetic.
"""

import json
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3
from tests import _codec_sweep
from tests.exact import round_to_binary

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode_all() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_all_codes_matches_torch_float8():
    ours = e4m3.decode(np.arange(256))
    ref = torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # signed zeros are kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_page_facts_range_and_field_widths():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["e4m3"]
    vals = e4m3.decode(np.arange(256))
    assert np.nanmax(vals) == facts["max_abs"] == e4m3.E4M3_MAX
    assert np.nanmin(vals) == -facts["max_abs"]
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    # 2^(exponent bits + mantissa bits + sign) codes, of which only the all-ones pattern is NaN
    assert 2 ** (1 + facts["exponent_bits"] + facts["mantissa_bits"]) == 256
    assert np.count_nonzero(np.isnan(vals)) == 2
    # each binade holds 2^mantissa_bits values
    pos = np.unique(vals[(~np.isnan(vals)) & (vals > 0)])
    for lo in (2.0 ** -6, 1.0, 2.0, 128.0):
        n = np.count_nonzero((pos >= lo) & (pos < 2 * lo))
        assert n == 2 ** facts["mantissa_bits"]


def test_nan_codes_and_count():
    vals = e4m3.decode(np.arange(256))
    assert set(np.flatnonzero(np.isnan(vals)).tolist()) == set(e4m3.NAN_CODES)
    assert e4m3.finite_codes().size == 254


def test_finite_values_are_multiples_of_2m9_and_roundtrip():
    c = e4m3.finite_codes()
    v = e4m3.decode(c)
    assert np.all(np.ldexp(v, 9) == np.rint(np.ldexp(v, 9)))
    back = e4m3.encode(v.astype(np.float32))
    assert np.array_equal(back, c)


def test_midpoints_round_to_even_code():
    c = np.arange(0x00, 0x7E, dtype=np.int64)  # non-negative neighbours (c, c + 1)
    lo, hi = e4m3.decode(c), e4m3.decode(c + 1)
    mid = (lo + hi) / 2  # exact: both have few significant bits
    assert np.all(mid.astype(np.float32).astype(np.float64) == mid)
    got = e4m3.encode(mid.astype(np.float32)).astype(np.int64)
    even = np.where(c % 2 == 0, c, c + 1)
    assert np.array_equal(got, even)
    # and negatives mirror it
    gotn = e4m3.encode((-mid).astype(np.float32)).astype(np.int64)
    assert np.array_equal(gotn, even | 0x80)


def test_encode_matches_exact_rational_rounding_on_samples():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x43E80001, size=4000, dtype=np.int64).astype(np.uint32)
    vals = bits.view(np.float32)
    got = e4m3.encode(vals)
    ref = torch_decode_all()
    table = {Fraction(float(ref[code])): code for code in range(0x7F)}  # non-negative codes
    for v, g in zip(vals.tolist(), got.tolist()):
        # E4M3 as a binary format: 4 significant bits, smallest normal exponent -6
        r = min(round_to_binary(Fraction(v), 4, -6), Fraction(448))
        assert table[r] == g


def test_saturation_and_specials():
    big = np.array([464.0001, 480.0, 1e6, 3.0e38, np.inf], dtype=np.float32)
    assert np.all(e4m3.encode(big) == 0x7E)
    assert np.all(e4m3.encode(-big) == 0xFE)
    nan = np.array([np.nan], dtype=np.float32)
    assert e4m3.encode(nan)[0] == 0x7F
    assert e4m3.encode(-nan)[0] == 0xFF
    assert e4m3.encode(np.array([-0.0], np.float32))[0] == 0x80
    assert e4m3.encode(np.array([np.float32(-1e-45)]))[0] == 0x80  # negative denormal -> -0


def test_encode_exhaustive_nonnegative_vs_torch():
    """Every non-negative float32 up to 464 (1,139,277,825 values) against torch's cast."""
    work = list(_codec_sweep.chunks())
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1),
                             mp_context=multiprocessing.get_context("spawn")) as ex:
        bad = sum(ex.map(_codec_sweep.mismatches_vs_torch, work))
    assert bad == 0


def test_encode_negative_sampled_vs_torch_and_sign_symmetry():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 0x43E80001, size=1 << 21, dtype=np.int64).astype(np.uint32)
    v = bits.view(np.float32)
    ours_neg = e4m3.encode(-v)
    ref_neg = torch.from_numpy(-v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours_neg, ref_neg)
    assert np.array_equal(ours_neg, e4m3.encode(v) | 0x80)


@pytest.mark.parametrize("lo_hi", [(0, 1 << 23), (0x3C000000, 0x3C000000 + (1 << 22))])
def test_encode_denormal_and_boundary_ranges_vs_torch(lo_hi):
    lo, hi = lo_hi
    bits = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(v), ref)
