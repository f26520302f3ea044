"""Pins for the oracle's dequantized fp64 GEMM and its grouped form (CPU only).

Independent references: exact rational sums (fractions.Fraction) on tiny shapes, exact int64
matmuls when every scale is 1 and every code decodes to an integer, exact rational rounding to
bf16 / float32, and special cases where the grouped GEMM reduces to the dense one.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm
from tests.exact import round_to_bf16, round_to_f32

TORCH_DEC = torch.arange(256, dtype=torch.int64).to(torch.uint8).view(torch.float8_e4m3fn).to(
    torch.float64).numpy()


def finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x7E), c).astype(np.uint8)


def random_scales(rng, shape):
    return (2.0 ** rng.uniform(-12, 2, size=shape)).astype(np.float32)


def exact_gemm(xq, sa, wq, sw):
    """Y[m][n] as exact Fractions, from torch's decoding of the codes."""
    M, K = xq.shape
    N = wq.shape[0]
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in TORCH_DEC]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (dec[xq[m, k]] * Fraction(float(sa[m, k // 128]))
                        * dec[wq[n, k]] * Fraction(float(sw[n // 128, k // 128])))
            out[m][n] = acc
    return out


@pytest.mark.parametrize("shape", [(3, 5, 128), (8, 8, 256), (1, 130, 256), (4, 2, 384)])
def test_fp64_gemm_vs_exact_rational(shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N + K)
    xq, wq = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa = random_scales(rng, (M, -(-K // 128)))
    sw = random_scales(rng, (-(-N // 128), -(-K // 128)))
    y = gemm.gemm_blockscaled(xq, sa, wq, sw, out="f64")
    ex = exact_gemm(xq, sa, wq, sw)
    A = np.abs(gemm.dequant_act(xq, sa))
    B = np.abs(gemm.dequant_weight(wq, sw))
    bound = (A @ B.T) * (K + 2) * 2.0 ** -52  # fp64 products and sums, any order
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= Fraction(bound[m, n])
    # the rounded outputs are the exact value rounded once (bf16) -- except at a rounding boundary
    yb = gemm.gemm_blockscaled(xq, sa, wq, sw, out="bf16")
    y32 = gemm.gemm_blockscaled(xq, sa, wq, sw, out="f32")
    for m in range(M):
        for n in range(N):
            rb = round_to_bf16(ex[m][n])
            got = Fraction(float(gemm.bf16_bits_to_f64(yb[m, n])))
            assert got == rb or abs(got - rb) <= abs(rb) * Fraction(1, 128)
            r32 = round_to_f32(ex[m][n])
            g32 = Fraction(float(y32[m, n]))
            assert g32 == r32 or abs(g32 - r32) <= abs(r32) * Fraction(1, 2 ** 23)


def test_integer_codes_unit_scales_equal_int64_matmul():
    """Codes whose values are integers (1..448) with S = 1: Y is an exact integer matmul."""
    ints = [c for c in range(0x38, 0x7F) if TORCH_DEC[c] == int(TORCH_DEC[c])]
    ints += [c | 0x80 for c in ints]
    rng = np.random.default_rng(5)
    M, N, K = 16, 256, 512
    xq = rng.choice(ints, size=(M, K)).astype(np.uint8)
    wq = rng.choice(ints, size=(N, K)).astype(np.uint8)
    sa = np.ones((M, K // 128), np.float32)
    sw = np.ones((N // 128, K // 128), np.float32)
    xi = TORCH_DEC[xq].astype(np.int64)
    wi = TORCH_DEC[wq].astype(np.int64)
    want = xi @ wi.T
    y = gemm.gemm_blockscaled(xq, sa, wq, sw, out="f64")
    assert np.array_equal(y, want.astype(np.float64))  # |Y| < 2^53: exact in fp64


def test_block_scales_apply_per_128_k_slice_and_row_block():
    """Scaling one K slice / one N block by 2 must double exactly that slice's contribution."""
    rng = np.random.default_rng(9)
    M, N, K = 4, 256, 384
    xq, wq = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa = np.ones((M, 3), np.float32)
    sw = np.ones((2, 3), np.float32)
    base = gemm.gemm_blockscaled(xq, sa, wq, sw)
    sa2 = sa.copy()
    sa2[1, 2] = 2.0
    d = gemm.gemm_blockscaled(xq, sa2, wq, sw) - base
    part = TORCH_DEC[xq[1, 256:]] @ TORCH_DEC[wq[:, 256:]].T
    assert np.array_equal(d[1], part) and np.all(np.delete(d, 1, axis=0) == 0)
    sw2 = sw.copy()
    sw2[1, 0] = 2.0
    d = gemm.gemm_blockscaled(xq, sa, wq, sw2) - base
    part = TORCH_DEC[xq[:, :128]] @ TORCH_DEC[wq[128:, :128]].T
    assert np.array_equal(d[:, 128:], part) and np.all(d[:, :128] == 0)


def test_bf16_rounding_vs_exact_and_torch():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -133, 2.0 ** -134,
                         3 * 2.0 ** -135, 1.5 * 2.0 ** -133, 2.0 ** -126 * (1 - 2.0 ** -9)]])
    bits = gemm.round_f64_to_bf16_bits(y)
    for v, b in zip(y.tolist(), bits.tolist()):
        want = round_to_bf16(Fraction(v))
        got = Fraction(float(gemm.bf16_bits_to_f64(np.array([b], np.uint16))[0]))
        assert got == want
    # on values that are float32-representable, torch's float32 -> bf16 cast is a single rounding
    y32 = y.astype(np.float32)
    y32 = y32[np.isfinite(y32)]
    ours = gemm.round_f64_to_bf16_bits(y32.astype(np.float64))
    ref = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_tolerance_sanity_against_exact():
    """The oracle's own rounded outputs sit well inside the parity tolerance of the exact sum."""
    rng = np.random.default_rng(17)
    M, N, K = 6, 128, 256
    xq, wq = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa, sw = random_scales(rng, (M, 2)), random_scales(rng, (1, 2))
    ex = np.array([[float(v) for v in row] for row in exact_gemm(xq, sa, wq, sw)])
    rms = np.sqrt(np.mean(ex ** 2))
    yb = gemm.bf16_bits_to_f64(gemm.gemm_blockscaled(xq, sa, wq, sw, out="bf16"))
    assert np.all(np.abs(yb - ex) <= 2.0 ** -7 * np.abs(ex) + 1e-3 * rms)
    y32 = gemm.gemm_blockscaled(xq, sa, wq, sw, out="f32").astype(np.float64)
    assert np.all(np.abs(y32 - ex) <= 1e-5 * rms)


def test_grouped_special_cases_reduce_to_dense():
    rng = np.random.default_rng(23)
    M, N, K, E = 50, 256, 256, 5
    xq = finite_codes(rng, (M, K))
    sa = random_scales(rng, (M, 2))
    wq1 = finite_codes(rng, (N, K))
    sw1 = random_scales(rng, (2, 2))
    dense = gemm.gemm_blockscaled(xq, sa, wq1, sw1)
    # one expert owning every row
    one = gemm.grouped_gemm_blockscaled(xq, sa, wq1[None], sw1[None], [0, M])
    assert np.array_equal(one, dense)
    # E identical experts, arbitrary segment boundaries (including empty experts)
    off = [0, 0, 17, 17, 49, 50]
    same = gemm.grouped_gemm_blockscaled(xq, sa, np.repeat(wq1[None], E, 0),
                                         np.repeat(sw1[None], E, 0), off)
    # equal up to the fp64 summation order BLAS picks for each segment height
    bound = (np.abs(gemm.dequant_act(xq, sa)) @ np.abs(gemm.dequant_weight(wq1, sw1)).T) * K * 2.0 ** -51
    assert np.all(np.abs(same - dense) <= bound)


def test_grouped_exact_rational_tiny():
    rng = np.random.default_rng(29)
    M, N, K, E = 7, 128, 128, 3
    xq = finite_codes(rng, (M, K))
    sa = random_scales(rng, (M, 1))
    wq = finite_codes(rng, (E, N, K))
    sw = random_scales(rng, (E, 1, 1))
    off = [0, 2, 2, 7]
    y = gemm.grouped_gemm_blockscaled(xq, sa, wq, sw, off)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ex = exact_gemm(xq[lo:hi], sa[lo:hi], wq[e], sw[e])
        for i in range(hi - lo):
            for n in range(0, N, 7):
                assert abs(Fraction(y[lo + i, n]) - ex[i][n]) <= abs(ex[i][n]) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 200)


def test_grouped_rejects_bad_offsets():
    xq = np.zeros((4, 128), np.uint8)
    sa = np.ones((4, 1), np.float32)
    wq = np.zeros((2, 128, 128), np.uint8)
    sw = np.ones((2, 1, 1), np.float32)
    for off in ([1, 2, 4], [0, 3, 2], [0, 2, 5]):
        with pytest.raises(ValueError):
            gemm.grouped_gemm_blockscaled(xq, sa, wq, sw, off)


def test_decode_used_by_gemm_is_the_codec():
    assert np.array_equal(np.nan_to_num(e4m3.decode(np.arange(256)), nan=7.0),
                          np.nan_to_num(TORCH_DEC, nan=7.0))
