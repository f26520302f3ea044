"""Pins for the oracle's 128x128 weight and 1x128 activation quantizers (CPU only).

Independent references: a group worked by hand from the pages' scale rule (golden fixture),
exact rational arithmetic for both IEEE float32 divisions, closed forms (power-of-two scales,
constant and single-element blocks) and invariants that any correct implementation satisfies.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import e4m3, quant
from tests.exact import bf16_bits_to_fraction, f32_to_fraction, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(values) -> np.ndarray:
    """Exactly-representable float values -> bf16 bit patterns (uint16)."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    back = t.to(torch.float32).numpy()
    assert np.array_equal(back.view(np.uint32), np.asarray(values, np.float32).view(np.uint32))
    return t.view(torch.int16).numpy().view(np.uint16)


def random_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ hand-worked group


def test_worked_group_activation_and_weight():
    d = json.load(open(os.path.join(GOLDEN, "worked_group.json")))
    x = np.zeros(128, dtype=np.float32)
    want = np.zeros(128, dtype=np.uint8)
    for e in d["entries"]:
        x[e["idx"]] = np.float32(float(e["x"]))
        want[e["idx"]] = int(e["code"], 16)
    bits = bf16_bits(x)
    q, sa = quant.quant_act_tok128(bits[None, :])
    assert sa.shape == (1, 1) and sa[0, 0] == np.float32(d["scale"])
    assert np.array_equal(q[0], want)
    # the same values as row 5 of an otherwise-zero 128x128 weight block
    w = np.zeros((128, 128), dtype=np.uint16)
    w[5] = bits
    wq, sw = quant.quant_weight_blk128(w)
    assert sw.shape == (1, 1) and sw[0, 0] == np.float32(d["scale"])
    assert np.array_equal(wq[5], want)
    assert np.all(np.delete(wq, 5, axis=0) == 0)


def test_page_granularity_shapes():
    g = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["granularity"]
    bw, bk = g["weight_block"]
    ga, gk = g["activation_group"]
    w = random_bf16((3 * bw, 2 * bk), 3, 0.02)
    _, sw = quant.quant_weight_blk128(w)
    assert sw.shape == (3, 2) and sw.dtype == np.float32
    x = random_bf16((5 * ga, 3 * gk), 4)
    _, sa = quant.quant_act_tok128(x)
    assert sa.shape == (5, 3) and sa.dtype == np.float32


# ------------------------------------------------------------------ IEEE divisions, exactly


def _exact_scale(amax_bits):
    a = bf16_bits_to_fraction(int(amax_bits) & 0x7FFF)
    if a == 0:
        return Fraction(1)
    return round_to_f32(a / 448)


def test_scale_is_correctly_rounded_f32_quotient():
    rng = np.random.default_rng(11)
    # normal and subnormal bf16 magnitudes, plus the extremes
    bits = np.concatenate([
        rng.integers(1, 0x7F80, size=3000), np.arange(1, 128), [0, 1, 0x7F7F, 0x0080, 0x007F]
    ]).astype(np.uint16)
    amax32 = quant.bf16_bits_to_f32(bits)
    S = quant.scale_from_amax(amax32)
    for b, s in zip(bits.tolist(), S.tolist()):
        assert f32_to_fraction(s) == _exact_scale(b)
        assert s > 0


def test_element_quotient_is_correctly_rounded_f32():
    rng = np.random.default_rng(12)
    for trial in range(40):
        # some groups with tiny (subnormal-S) amax, some ordinary
        scale = float(2.0 ** rng.integers(-140, 10))
        xb = random_bf16((128,), 100 + trial, scale)
        x32 = quant.bf16_bits_to_f32(xb)
        if not np.all(np.isfinite(x32)) or np.max(np.abs(x32)) == 0:
            continue
        q, S = quant.quantize_group(x32)
        Sf = f32_to_fraction(float(S))
        for xv, code in zip(x32.tolist(), q.tolist()):
            t = round_to_f32(Fraction(xv) / Sf)  # S > 0: the quotient keeps x's sign
            t32 = np.float32(np.copysign(float(t), xv))
            assert e4m3.encode(np.array([t32]))[0] == code


# ------------------------------------------------------------------ closed forms


@pytest.mark.parametrize("j", [-20, -7, -1, 0, 1, 5, 12])
def test_power_of_two_scale_closed_form(j):
    """amax = 448 * 2^j gives S = 2^j exactly, and E4M3-grid values times 2^j decode back exactly."""
    grid = e4m3.decode(e4m3.finite_codes())
    rng = np.random.default_rng(j + 50)
    vals = rng.choice(grid, size=(128, 128))
    vals[:, 0] = 448.0  # every row (activation group) and the block reach amax = 448 * 2^j
    x = np.ldexp(vals, j).astype(np.float32)
    bits = bf16_bits(x.reshape(-1)).reshape(128, 128)  # <= 4 significant bits: bf16 holds them
    wq, sw = quant.quant_weight_blk128(bits)
    assert sw[0, 0] == np.float32(2.0 ** j)
    assert np.array_equal(e4m3.decode(wq), vals)
    xq, sa = quant.quant_act_tok128(bits)
    assert np.all(sa == np.float32(2.0 ** j))
    assert np.array_equal(e4m3.decode(xq), vals)


@pytest.mark.parametrize("c", [0.02, -1.5, 3.0e-5, 1.0e30, 9.0e-40])
def test_constant_block_maps_to_vmax(c):
    b = torch.tensor([c], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    bits = np.full((128, 128), b[0].view(np.uint16))
    wq, sw = quant.quant_weight_blk128(bits)
    want = 0xFE if c < 0 else 0x7E
    assert np.all(wq == want)
    xq, sa = quant.quant_act_tok128(bits[:3])
    assert np.all(xq == want)


def test_single_nonzero_block_and_zero_block():
    w = np.zeros((256, 128), dtype=np.uint16)
    w[7, 9] = bf16_bits([-0.375])[0]
    w[128 + 3, 1] = 0x8000  # -0.0 in an otherwise zero block
    wq, sw = quant.quant_weight_blk128(w)
    assert wq[7, 9] == 0xFE
    assert np.count_nonzero(wq[:128]) == 1
    assert sw[0, 0] == np.float32(np.float32(0.375) / np.float32(448))
    assert sw[1, 0] == 1.0  # amax == 0 -> S = 1
    assert wq[128 + 3, 1] == 0x80 and np.count_nonzero(wq[128:]) == 1


def test_ragged_edges_use_in_range_elements_only():
    x = random_bf16((3, 300), 21)
    q, sa = quant.quant_act_tok128(x)
    assert sa.shape == (3, 3)
    tail = quant.bf16_bits_to_f32(x[:, 256:])
    want = quant.scale_from_amax(np.max(np.abs(tail), axis=1))
    assert np.array_equal(sa[:, 2], want)
    w = random_bf16((200, 130), 22, 0.02)
    wq, sw = quant.quant_weight_blk128(w)
    assert sw.shape == (2, 2)
    corner = quant.bf16_bits_to_f32(w[128:, 128:])
    assert sw[1, 1] == quant.scale_from_amax(np.max(np.abs(corner)))


def test_nonfinite_input_rejected():
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        quant.quant_act_tok128(x)
    x[0, 3] = 0x7FC1  # NaN
    with pytest.raises(ValueError):
        quant.quant_weight_blk128(np.tile(x, (128, 1)))


# ------------------------------------------------------------------ invariants (property tests)

group_bits = st.lists(st.integers(0, 0xFFFF).filter(lambda b: (b & 0x7F80) != 0x7F80),
                      min_size=128, max_size=128)


@settings(max_examples=150, deadline=None)
@given(group_bits)
def test_invariants_on_arbitrary_groups(bits):
    xb = np.array(bits, dtype=np.uint16)
    x32 = quant.bf16_bits_to_f32(xb)
    q, sa = quant.quant_act_tok128(xb[None, :])
    q, S = q[0], sa[0, 0]
    amax = np.max(np.abs(x32))
    if amax == 0:
        assert S == 1.0 and np.all((q & 0x7F) == 0)
        return
    # the amax element(s) map to +-448
    for i in np.flatnonzero(np.abs(x32) == amax):
        assert q[i] == (0xFE if x32[i] < 0 else 0x7E)
    # sign symmetry and permutation invariance
    qn, san = quant.quant_act_tok128((xb ^ 0x8000)[None, :])
    assert san[0, 0] == S and np.array_equal(qn[0], q ^ 0x80)
    perm = np.random.default_rng(len(bits)).permutation(128)
    qp, sap = quant.quant_act_tok128(xb[perm][None, :])
    assert sap[0, 0] == S and np.array_equal(qp[0], q[perm])
    # rounding error bound: half a step of the E4M3 grid at the decoded value, plus the one
    # float32 rounding of the quotient
    t = (x32 / S).astype(np.float64)
    d = e4m3.decode(q)
    e = np.floor(np.log2(np.maximum(np.abs(d), 2.0 ** -6)))
    half_step = np.ldexp(1.0, (e - 4).astype(np.int64))
    assert np.all(np.abs(t - d) <= half_step * (1 + 2.0 ** -20) + np.abs(t) * 2.0 ** -23)
    # re-quantizing the dequantized values with the same (normal) S returns the same codes
    if S >= np.float32(2.0 ** -126):
        deq = (d * np.float64(S)).astype(np.float32)
        assert np.array_equal(e4m3.encode((deq / S).astype(np.float32)), q)


def test_concatenation_along_n_keeps_codes():
    a = random_bf16((256, 384), 31, 0.02)
    b = random_bf16((128, 384), 32, 0.02)
    qa, sa_ = quant.quant_weight_blk128(a)
    qb, sb = quant.quant_weight_blk128(b)
    qc, sc = quant.quant_weight_blk128(np.concatenate([a, b]))
    assert np.array_equal(qc, np.concatenate([qa, qb]))
    assert np.array_equal(sc, np.concatenate([sa_, sb]))


def test_activation_rows_are_independent():
    x = random_bf16((6, 512), 41)
    q, sa = quant.quant_act_tok128(x)
    for r in range(6):
        qr, sr = quant.quant_act_tok128(x[r:r + 1])
        assert np.array_equal(qr[0], q[r]) and np.array_equal(sr[0], sa[r])
