"""Accuracy of the two block-scale formats against the unquantized product (the comparison the
NeMo RL blog's advanced options and Unified FP8's "FP8 scale choice" section call for: FP32
scales against power-of-two, E8M0-representable ones).

For the configurations' layer shapes, on their seeded synthetic tensors (weights N(0, 0.02), with
0.1 % x10 outliers for the dense models, activations N(0, 1) with 1 % x20 outlier channels), the
oracle quantizes X (1x128 groups) and W (128x128 blocks) with each scale format and forms the
exact float64 GEMM of the dequantized operands; the reference is the exact float64 product of the
bf16 operands themselves. Reported per shape and format: the relative Frobenius error
||Y_q - Y|| / ||Y|| and the largest element error over rms(Y). The checks are the ones the
number format fixes: E4M3 keeps 3 mantissa bits, so a normal quotient is off by at most 2^-4 of
itself, and the relative error of the product of two such operands stays below a few 2^-4; a
power-of-two scale maps a group's amax into [224, 448] instead of onto 448, so its error is not
below the FP32 scale's by more than noise, and not above it by more than the one binade it gives
up. The numbers printed here (pytest -s) are the table of the design notes.
"""

import numpy as np
import pytest
import torch

from oracle import gemm as og
from oracle import quant as oq
from workloads import synth

SHAPES = [
    # (label, M, N, K, weight outliers)
    ("Qwen3-8B q_proj, M=64", 64, 4096, 4096, 0.001),
    ("Qwen3-8B down_proj, M=64", 64, 4096, 12288, 0.001),
    ("Qwen3-8B gate_proj, 256 prefill rows", 256, 12288, 4096, 0.001),
    ("Llama-3.1-8B up_proj, M=256", 256, 14336, 4096, 0.001),
    ("Qwen3-30B-A3B expert gate/up, 256 rows", 256, 1536, 2048, 0.0),
]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def errors(M, N, K, w_out, seed):
    x = synth.act_bf16(M, K, seed=seed)
    w = synth.weight_bf16(N, K, seed=seed + 1, outlier_frac=w_out)
    xb, wb = _bits(x), _bits(w)
    ref = oq.bf16_bits_to_f32(xb).astype(np.float64) @ oq.bf16_bits_to_f32(wb).astype(np.float64).T
    rms = float(np.sqrt(np.mean(ref ** 2)))
    out = {}
    for scale in ("fp32", "pow2"):
        xq, sa = oq.quant_act_tok128(xb, scale=scale)
        wq, sw = oq.quant_weight_blk128(wb, scale=scale)
        y = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
        d = y - ref
        out[scale] = (float(np.linalg.norm(d) / np.linalg.norm(ref)), float(np.abs(d).max() / rms))
    return out


@pytest.mark.parametrize("label,M,N,K,w_out", SHAPES)
def test_power_of_two_against_fp32_scales(label, M, N, K, w_out):
    e = errors(M, N, K, w_out, seed=synth.seed_of(70, N, K))
    (f_rel, f_max), (p_rel, p_max) = e["fp32"], e["pow2"]
    print(f"\n| {label} | {f_rel:.3e} | {p_rel:.3e} | {p_rel / f_rel:.3f} | {f_max:.3e} | "
          f"{p_max:.3e} |")
    # both within what 3 mantissa bits allow for the product of two quantized operands
    assert f_rel < 2.0 ** -4 and p_rel < 2.0 ** -4
    # giving up at most one binade of each group's range costs at most a factor of 2 in error,
    # and a power-of-two scale is never the more accurate one by more than noise
    assert 0.95 < p_rel / f_rel < 2.0


def test_power_of_two_equals_fp32_where_amax_is_448_times_a_power_of_two():
    """Where every group's amax / 448 is a power of two the two formats quantize identically,
    so their errors against the unquantized product are the same (a check that the comparison
    above measures the scale format and nothing else)."""
    rng = np.random.default_rng(5)
    M, N, K = 32, 256, 512
    x = np.clip(rng.standard_normal((M, K)).astype(np.float32), -6.0, 6.0)
    w = np.clip(rng.standard_normal((N, K)).astype(np.float32) * 0.02, -0.1, 0.1)
    # every 1x128 group / 128x128 block reaches exactly 448 * 2^e (7 = 448 * 2^-6, 0.109375 =
    # 448 * 2^-12, both exact in bf16) in its first element, and nothing exceeds it
    for g in range(K // 128):
        x[:, 128 * g] = np.where(x[:, 128 * g] < 0, -7.0, 7.0)
        for b in range(N // 128):
            w[128 * b, 128 * g] = 448.0 * 2.0 ** -12
    xb = torch.from_numpy(x).to(torch.bfloat16)
    wb = torch.from_numpy(w).to(torch.bfloat16)
    res = {}
    for scale in ("fp32", "pow2"):
        xq, sa = oq.quant_act_tok128(_bits(xb), scale=scale)
        wq, sw = oq.quant_weight_blk128(_bits(wb), scale=scale)
        res[scale] = (xq, sa, wq, sw)
    for a, b in zip(res["fp32"], res["pow2"]):
        assert np.array_equal(a, b)
