"""Blockscaled FP8 GEMM and its grouped-expert form, as fp64 sums. TEST INFRASTRUCTURE.

Definition (NeMo RL blog, "FP8 for linear layers in RL", Table 1 and the sentence after it: the
linear layer runs its product on the FP8 operands with FP32 block scales; Unified FP8 blog,
"KL attribution" section: the "fake quant" view, i.e. quantize, dequantize, then multiply in high
precision): with the dequantized operands

    A[m, k] = dec(Xq[m, k]) * sa[m, k // 128]
    B[n, k] = dec(Wq[n, k]) * sw[n // 128, k // 128]

the layer output is Y = A @ B^T. Here A and B are built exactly in float64 (a <= 4-bit
significand times a 24-bit one), the product is one float64 matmul, and the result is rounded
once, to nearest even, to the output type (bf16 or float32).

The grouped form (mixture-of-experts expert layers, quantized like linears per the FP8-RL
write-up, section 1): rows off[e] .. off[e+1]-1 of Xq use expert e's Wq[e] and sw[e]; the row
order is kept.
"""

from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 128


def dequant_act(xq, sa) -> np.ndarray:
    """A[m, k] = dec(Xq[m, k]) * sa[m, k // 128], float64."""
    xq = np.asarray(xq, dtype=np.uint8)
    sa = np.asarray(sa, dtype=np.float32)
    M, K = xq.shape
    scale = np.repeat(sa.astype(np.float64), BLOCK, axis=1)[:, :K]
    return e4m3.decode(xq) * scale


def dequant_weight(wq, sw) -> np.ndarray:
    """B[n, k] = dec(Wq[n, k]) * sw[n // 128, k // 128], float64."""
    wq = np.asarray(wq, dtype=np.uint8)
    sw = np.asarray(sw, dtype=np.float32)
    N, K = wq.shape
    scale = np.repeat(np.repeat(sw.astype(np.float64), BLOCK, axis=0), BLOCK, axis=1)[:N, :K]
    return e4m3.decode(wq) * scale


def round_f64_to_bf16_bits(y) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) in one step; returns uint16 bits.

    bf16 keeps 8 significant bits; its normal range starts at 2^-126 and its subnormals are
    multiples of 2^-133. Magnitudes that round above the largest finite bf16 become infinity.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("non-finite GEMM result")
    _, ex = np.frexp(y)  # |y| = f * 2^ex with f in [0.5, 1)
    step_exp = np.maximum(ex - 8, -133)  # weight of the last kept bit
    r = np.ldexp(np.rint(np.ldexp(y, -step_exp)), step_exp)  # rint: half to even
    r32 = r.astype(np.float32)  # exact: r has <= 8 significant bits (or overflows to inf)
    bits = r32.view(np.uint32)
    if np.any((bits & 0xFFFF) != 0):
        raise AssertionError("bf16 rounding left low bits set")
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gemm_blockscaled(xq, sa, wq, sw, out: str = "f64"):
    """Y = A @ B^T in float64, returned as float64 ('f64'), float32 ('f32') or bf16 bits ('bf16')."""
    A = dequant_act(xq, sa)
    B = dequant_weight(wq, sw)
    if A.shape[1] != B.shape[1]:
        raise ValueError("K mismatch")
    y = A @ B.T
    return _finish(y, out)


def grouped_gemm_blockscaled(xq, sa, wq, sw, offsets, out: str = "f64"):
    """Per-expert blockscaled GEMM over the row segments given by ``offsets`` (length E + 1)."""
    xq = np.asarray(xq, dtype=np.uint8)
    off = np.asarray(offsets, dtype=np.int64)
    E = off.size - 1
    wq = np.asarray(wq)
    if wq.ndim != 3 or wq.shape[0] != E:
        raise ValueError("wq must be [E][N][K]")
    if off[0] != 0 or off[-1] != xq.shape[0] or np.any(np.diff(off) < 0):
        raise ValueError("offsets must start at 0, be nondecreasing and end at M_total")
    N = wq.shape[1]
    y = np.zeros((xq.shape[0], N), dtype=np.float64)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            y[lo:hi] = gemm_blockscaled(xq[lo:hi], sa[lo:hi], wq[e], sw[e], out="f64")
    return _finish(y, out)


def _finish(y, out):
    if out == "f64":
        return y
    if out == "f32":
        return y.astype(np.float32)
    if out == "bf16":
        return round_f64_to_bf16_bits(y)
    raise ValueError(f"unknown output type {out!r}")
