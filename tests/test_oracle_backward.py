"""Pins for the oracle's FP8 backward pass (Dgrad, Wgrad; CPU only).

Independent references: the hand-worked 1x128 group placed as a column (128x1 group), transpose
symmetry of 128x128 block quantization checked element by element against the forward quantizer,
a direct Dgrad sum over the untransposed weight codes written as exact Fractions, the row-scaled
GEMM against exact Fractions and against the blockwise GEMM where the two definitions coincide,
and the FP8 gradients against the exact bf16 gradients within the quantization error bound.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import backward, e4m3, gemm, quant
from tests.test_oracle_gemm import finite_codes, random_scales
from tests.test_oracle_quant import bf16_bits, random_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_group_as_a_column():
    d = json.load(open(os.path.join(GOLDEN, "worked_group.json")))
    col = np.zeros(128, dtype=np.float32)
    want = np.zeros(128, dtype=np.uint8)
    for e in d["entries"]:
        col[e["idx"]] = float(e["x"])
        want[e["idx"]] = int(e["code"], 16)
    x = np.zeros((128, 3), dtype=np.float32)
    x[:, 1] = col
    x[:, 0] = 1.0
    xt_q, st = backward.quant_colwise128(bf16_bits(x.ravel()).reshape(128, 3))
    assert xt_q.shape == (3, 128) and st.shape == (3, 1)
    assert np.array_equal(xt_q[1], want)
    assert st[1, 0] == np.float32(d["scale"])
    assert st[0, 0] == np.float32(1.0) / np.float32(448.0) and np.all(xt_q[0] == 0x7E)
    assert st[2, 0] == 1.0 and np.all(xt_q[2] == 0)  # an all-zero column


@pytest.mark.parametrize("N,K", [(256, 384), (130, 200), (128, 128), (300, 129)])
def test_weight_transpose_symmetry(N, K):
    w = random_bf16((N, K), seed=N + K, scale=0.02)
    wq, sw = quant.quant_weight_blk128(w)
    wqt, swt = backward.quant_weight_blk128_t(w)
    assert wqt.shape == (K, N) and swt.shape == sw.T.shape
    for n in range(0, N, 37):
        for k in range(0, K, 29):
            assert wqt[k, n] == wq[n, k]
            assert swt[k // 128, n // 128] == sw[n // 128, k // 128]
    assert np.array_equal(wqt, wq.T) and np.array_equal(swt, sw.T)


def test_colwise_is_rowwise_of_transpose_per_element():
    x = random_bf16((256, 5), seed=9)
    xt_q, st = backward.quant_colwise128(x)
    x32 = quant.bf16_bits_to_f32(x)
    for k in range(5):
        for mb in range(2):
            grp = x32[128 * mb:128 * (mb + 1), k]
            S = np.float32(np.max(np.abs(grp)) / np.float32(448.0))
            assert st[k, mb] == S
            assert np.array_equal(xt_q[k, 128 * mb:128 * (mb + 1)], e4m3.encode((grp / S).astype(np.float32)))


def _exact_dgrad(dyq, s_dy, wq, sw):
    """dX[m][k] = sum_n s_dy[m][n/128] sw[n/128][k/128] dec(dYq[m][n]) dec(Wq[n][k]), directly over
    the forward weight codes (no transposed copy), as exact Fractions."""
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.decode(np.arange(256))]
    M, N = dyq.shape
    K = wq.shape[1]
    out = [[Fraction(0)] * K for _ in range(M)]
    for m in range(M):
        for k in range(K):
            acc = Fraction(0)
            for n in range(N):
                acc += (Fraction(float(s_dy[m, n // 128])) * Fraction(float(sw[n // 128, k // 128]))
                        * dec[dyq[m, n]] * dec[wq[n, k]])
            out[m][k] = acc
    return out


def test_dgrad_through_transposed_copy_equals_direct_sum():
    M, N, K = 128, 256, 130
    dy = random_bf16((M, N), seed=1, scale=1e-3)
    x = random_bf16((M, K), seed=2)
    w = random_bf16((N, K), seed=3, scale=0.02)
    dx, _ = backward.linear_backward_fp8(dy, x, w)
    dyq, s_dy = quant.quant_act_tok128(dy[:3])
    wq, sw = quant.quant_weight_blk128(w)
    ex = _exact_dgrad(dyq, s_dy, wq, sw)
    for m in range(3):
        for k in range(0, K, 7):
            assert abs(Fraction(dx[m, k]) - ex[m][k]) <= abs(ex[m][k]) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 120)


def test_rowscaled_gemm_vs_exact_rational():
    rng = np.random.default_rng(4)
    M, N, K = 3, 4, 256
    aq, bq = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa, sb = random_scales(rng, (M, 2)), random_scales(rng, (N, 2))
    y = backward.gemm_rowscaled(aq, sa, bq, sb)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.decode(np.arange(256))]
    for m in range(M):
        for n in range(N):
            ex = sum(Fraction(float(sa[m, k // 128])) * Fraction(float(sb[n, k // 128])) * dec[aq[m, k]]
                     * dec[bq[n, k]] for k in range(K))
            bound = sum(abs(Fraction(float(sa[m, k // 128])) * Fraction(float(sb[n, k // 128])) * dec[aq[m, k]]
                            * dec[bq[n, k]]) for k in range(K)) * Fraction(K + 2, 2 ** 52)
            assert abs(Fraction(y[m, n]) - ex) <= bound


def test_rowscaled_equals_blockscaled_when_row_scales_are_blockwise():
    rng = np.random.default_rng(5)
    M, N, K = 5, 256, 384
    aq, bq = finite_codes(rng, (M, K)), finite_codes(rng, (N, K))
    sa = random_scales(rng, (M, 3))
    sw = random_scales(rng, (2, 3))
    sb = np.repeat(sw, 128, axis=0)  # every row of a 128-row block carries the block's scale
    assert np.array_equal(backward.gemm_rowscaled(aq, sa, bq, sb, out="bf16"),
                          gemm.gemm_blockscaled(aq, sa, bq, sw, out="bf16"))


def test_gradients_close_to_exact_bf16_gradients():
    # each operand's codes are within 2^-4 relative (half an E4M3 step) of the bf16 value, or
    # within 2^-10 S for subnormal codes: the FP8 gradients sit within that of the exact ones
    M, N, K = 256, 256, 128
    dy = random_bf16((M, N), seed=11, scale=1e-2)
    x = random_bf16((M, K), seed=12)
    w = random_bf16((N, K), seed=13, scale=0.02)
    dx, dw = backward.linear_backward_fp8(dy, x, w)
    f = lambda b: quant.bf16_bits_to_f32(b).astype(np.float64)
    dx_ex = f(dy) @ f(w)
    dw_ex = f(dy).T @ f(x)
    mag_dx = np.abs(f(dy)) @ np.abs(f(w))
    mag_dw = np.abs(f(dy)).T @ np.abs(f(x))
    assert np.all(np.abs(dx - dx_ex) <= 2 * 2.0 ** -4 * mag_dx * 1.07 + 1e-9)
    assert np.all(np.abs(dw - dw_ex) <= 2 * 2.0 ** -4 * mag_dw * 1.07 + 1e-9)
    # and against torch's own float64 products of the same inputs
    t = lambda b: torch.from_numpy(f(b))
    assert np.allclose(dw_ex, (t(dy).T @ t(x)).numpy())


def test_rowscaled_rejects_k_mismatch():
    with pytest.raises(ValueError):
        backward.gemm_rowscaled(np.zeros((2, 128), np.uint8), np.ones((2, 1), np.float32),
                                np.zeros((2, 256), np.uint8), np.ones((2, 2), np.float32))
