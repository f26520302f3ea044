"""Blockwise (128x128) weight and per-token (1x128) activation quantizers. TEST INFRASTRUCTURE.

Follows, step by step:

* Unified FP8 (LMSYS blog), quick-read section, the two quantization equations: the scale of a
  group X is S = max|X| / V_max and each element becomes Q(x) = round(x / S), V_max being the
  largest FP8 value (448 for E4M3, per the FP8-RL write-up, section 1);
* the same blog's "FP8 scale choice" section and the NeMo RL blog's Table 1: S is an FP32 number;
* FP8-RL write-up, section 1, and NeMo RL Table 1: weights use one scale per 128x128 block,
  recomputed each time the weights change; activations use one scale per 1x128 group of a token
  row, computed from the live values.

Readings where the pages leave a step open (each also listed in the design notes):

* Q2/Q6: S is the float32 quotient fp32(amax / 448) by IEEE division (stored as S, not 1/S), and
  the element quotient fp32(x) / S is an IEEE float32 division;
* Q3: a group whose amax is 0 gets S = 1 (all its codes are then signed zeros);
* Q4/Q5: "round" is round-to-nearest-even onto the E4M3 grid, saturating at +-448;
* Q7: a ragged edge block/group takes its amax over its in-range elements only;
* Q8/Q9: weights are W[N][K] (out x in) with block (i, j) covering rows 128i.. and columns 128j..;
  scales are sw[ceil(N/128)][ceil(K/128)] row-major; activation groups are 128 consecutive K
  elements of one row of X[M][K], scales sa[M][ceil(K/128)] row-major;
* Q12: non-finite inputs are outside the contract and raise ValueError.

Power-of-two scales (the NeMo RL blog's advanced FP8 options, which switch the weight and
activation scaling factors from FP32 to powers of 2; Unified FP8's "FP8 scale choice" section
contrasts FP32 scales with power-of-two E8M0 ones). Reading Q13: S is the smallest power of two
not below amax / 448 -- so no element leaves [-448, 448] -- but at least 2^-127, the smallest
E8M0 value; amax == 0 gives S = 1. The element step is unchanged: fp32(x) / S, which is exact
unless the quotient is below the float32 normal range.
"""

from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 128
V_MAX = np.float32(e4m3.E4M3_MAX)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16 / int16) to float32."""
    b = np.asarray(bits)
    if b.dtype not in (np.uint16, np.int16):
        raise TypeError("bf16 input must be given as 16-bit bit patterns")
    return (b.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _check_finite(x32: np.ndarray) -> None:
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite input is outside the quantizer's contract")


def scale_from_amax(amax) -> np.ndarray:
    """S = fp32(amax / 448) by IEEE float32 division; S = 1 where amax == 0."""
    a = np.asarray(amax, dtype=np.float32)
    s = (a / V_MAX).astype(np.float32)
    return np.where(a == np.float32(0), np.float32(1.0), s).astype(np.float32)


POW2_MIN_EXP = -127  # 2^-127: the smallest E8M0 scale


def scale_from_amax_pow2(amax) -> np.ndarray:
    """Q13: S = 2^e, e the least integer with 448 * 2^e >= amax (exact, from frexp), e >= -127;
    S = 1 where amax == 0."""
    a = np.asarray(amax, dtype=np.float64)  # float32 amax widens exactly
    f, E = np.frexp(a)                       # a = f * 2^E, f in [0.5, 1)
    # 448 = 0.875 * 2^9:  448 * 2^e >= f * 2^E  <=>  2^(e + 9 - E) >= f / 0.875
    e = E - 9 + (f > 0.875)
    e = np.maximum(e, POW2_MIN_EXP)
    s = np.ldexp(np.float64(1.0), e).astype(np.float32)
    return np.where(a == 0.0, np.float32(1.0), s).astype(np.float32)


SCALES = {"fp32": scale_from_amax, "pow2": scale_from_amax_pow2}


def _scale_fn(scale: str):
    if scale not in SCALES:
        raise ValueError(f"scale must be one of {sorted(SCALES)}")
    return SCALES[scale]


def quantize_group(x32: np.ndarray, scale: str = "fp32"):
    """Quantize one group (any shape) of float32 values: returns (codes uint8, S float32)."""
    x32 = np.asarray(x32, dtype=np.float32)
    _check_finite(x32)
    amax = np.max(np.abs(x32)) if x32.size else np.float32(0)
    S = _scale_fn(scale)(amax)
    q = e4m3.encode((x32 / S).astype(np.float32))
    return q, np.float32(S)


def quant_weight_blk128(w_bits, scale: str = "fp32"):
    """Weight W[N][K] (bf16 bits) -> (Wq uint8 [N][K], sw float32 [ceil(N/128)][ceil(K/128)]).
    `scale`: "fp32" (Q2) or "pow2" (Q13)."""
    x32 = bf16_bits_to_f32(w_bits)
    if x32.ndim != 2:
        raise ValueError("weight must be 2-D [N][K]")
    _check_finite(x32)
    N, K = x32.shape
    nb, kb = -(-N // BLOCK), -(-K // BLOCK)
    sw = np.empty((nb, kb), dtype=np.float32)
    q = np.empty((N, K), dtype=np.uint8)
    for i in range(nb):
        for j in range(kb):
            blk = x32[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK]
            q[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK], sw[i, j] = quantize_group(
                blk, scale)
    return q, sw


def quant_act_tok128(x_bits, scale: str = "fp32"):
    """Activation X[M][K] (bf16 bits) -> (Xq uint8 [M][K], sa float32 [M][ceil(K/128)]).
    `scale`: "fp32" (Q2) or "pow2" (Q13)."""
    scale_of = _scale_fn(scale)
    x32 = bf16_bits_to_f32(x_bits)
    if x32.ndim != 2:
        raise ValueError("activation must be 2-D [M][K]")
    _check_finite(x32)
    M, K = x32.shape
    kb = -(-K // BLOCK)
    sa = np.empty((M, kb), dtype=np.float32)
    q = np.empty((M, K), dtype=np.uint8)
    for j in range(kb):
        cols = x32[:, j * BLOCK:(j + 1) * BLOCK]  # every row's j-th group at once
        amax = np.max(np.abs(cols), axis=1) if cols.shape[1] else np.zeros(M, np.float32)
        S = scale_of(amax)
        sa[:, j] = S
        q[:, j * BLOCK:(j + 1) * BLOCK] = e4m3.encode((cols / S[:, None]).astype(np.float32))
    return q, sa
