"""GPU parity of the GEMM on bf16 activations (activation quantization fused in).

fp8rl_gemm_w8a8_fused_act_quant takes bf16 activations; its result must equal, within the GEMM
contract (|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref) for bf16 output, <= 1e-5 rms(ref) for float32
output with f16 slice sums), the oracle's GEMM of the oracle's 1x128 quantization of the same
activations, and be bit-identical to the library's two-launch path (quantize, then GEMM): up to
4 rows one kernel quantizes exactly as the quantizer does and multiplies in the blockscaled
GEMM's order, above that the call runs those two kernels itself. Inputs: seeded
synthetic activations (N(0, 1) with outlier channels) and weights of the decode shapes, larger
token counts on every GEMM path, plus edge rows.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import (assert_gemm_close, assert_within, bits16, fp8_slice_bound,
                            gemm_out_to_f64, to_dev_f32, to_dev_u8)
from workloads import synth

pytestmark = pytest.mark.gpu


def _weights(N, K, seed, scale="fp32"):
    w = synth.weight_bf16(N, K, seed=seed, outlier_frac=0.001)
    return oq.quant_weight_blk128(bits16(w), scale=scale)


def _check(x: torch.Tensor, wq, sw, what, scale="fp32", outs=("bf16", "f32"), accum=None):
    """x: bf16 on the GPU (any row pitch); wq / sw: oracle weight codes and scales."""
    M, K = x.shape
    N = wq.shape[0]
    print(f"[fused act gemm] {what} M={M} N={N} K={K} scale={scale} accum={accum}", flush=True)
    xq, sa = oq.quant_act_tok128(bits16(x), scale=scale)
    ref64 = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
    dwq, dsw = to_dev_u8(wq), to_dev_f32(sw)
    worst = {}
    for out in outs:
        dt = torch.bfloat16 if out == "bf16" else torch.float32
        y = fq.gemm_fused_act(x, dwq, dsw, out_dtype=dt, accum=accum, scale=scale)
        gxq, gsa = fq.quant_act(x, scale=scale)
        y_unfused = fq.gemm(gxq, gsa, dwq, dsw, out_dtype=dt, accum=accum)
        torch.cuda.synchronize()
        got = gemm_out_to_f64(y)
        if out == "bf16":
            ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
        else:
            ref = ref64.astype(np.float32).astype(np.float64)
        worst[out] = assert_gemm_close(got, ref, ref64, out, what)
        # the two-launch path: activation codes and scales bit-exact against the oracle (checked
        # elsewhere), the same GEMM kernel and slice order, hence the same bits
        assert torch.equal(y, y_unfused), what + " (two launches)"
    print(f"    worst err/bound {worst}", flush=True)


@pytest.mark.parametrize("M,N,K", [(64, 4096, 4096), (64, 6144, 4096), (64, 4096, 12288),
                                   (1, 128, 256), (3, 384, 768), (17, 256, 16384),
                                   (20, 512, 1024), (32, 2048, 2048), (33, 1024, 1280),
                                   (48, 12288, 4096), (8, 65664, 256), (64, 1024, 512),
                                   (16, 4096, 4096), (16, 2048, 384), (5, 8192, 1152),
                                   (2, 1024, 384), (4, 4096, 4096), (4, 6144, 12288),
                                   (65, 256, 384), (100, 1024, 4096), (300, 768, 2048),
                                   (256, 16384, 1024)])
def test_decode_shapes(M, N, K):
    x = synth.act_bf16(M, K, seed=synth.seed_of(60, M * 7919 + N, K)).cuda()
    _check(x, *_weights(N, K, synth.seed_of(61, N, K)), f"decode {M}x{N}x{K}")


def test_qwen3_gate_up_full_size():
    """Qwen3-8B gate/up (24576 x 4096) at M = 64, as the decode step runs it."""
    x = synth.act_bf16(64, 4096, seed=synth.seed_of(62, 0)).cuda()
    _check(x, *_weights(24576, 4096, synth.seed_of(62, 1)), "gate_up", outs=("bf16",))


def test_row_pitch_and_column_slice():
    big = synth.act_bf16(40, 6144, seed=synth.seed_of(63, 0)).cuda()
    wq, sw = _weights(1024, 4096, synth.seed_of(63, 1))
    _check(big[:, 1024:5120], wq, sw, "column slice of a wider activation")
    _check(big[::2, :4096], wq, sw, "every other row")


def test_edge_rows():
    """A zero row (scale 1), a row of huge values, tiny and subnormal values, one dominant
    outlier per group and rows whose groups differ in scale by 2^60."""
    M, K = 24, 2048
    x = synth.act_bf16(M, K, seed=synth.seed_of(64, 0))
    x[0] = 0.0
    x[1] = 1.0e30
    x[1, ::3] = -1.0e30
    x[2] *= 1e-38
    x[3] = torch.tensor(1e-40, dtype=torch.bfloat16)
    x[4, 7] = 1e4
    for g in range(K // 128):
        x[5, 128 * g:128 * (g + 1)] *= 2.0 ** (-30 + 4 * g)
    wq, sw = _weights(512, K, synth.seed_of(64, 1))
    _check(x.cuda(), wq, sw, "edge rows")


def test_edge_rows_single_kernel():
    """The one-kernel form (M <= 4): a zero row, a row of huge values, a bf16-subnormal row and
    groups 2^4 apart in scale with one dominant outlier."""
    M, K = 4, 2048
    x = synth.act_bf16(M, K, seed=synth.seed_of(68, 0))
    x[0] = 0.0
    x[1] = 1.0e30
    x[1, ::3] = -1.0e30
    x[2] = torch.tensor(1e-40, dtype=torch.bfloat16)
    x[3, 7] = 1e4
    for g in range(K // 128):
        x[3, 128 * g:128 * (g + 1)] *= 2.0 ** (-30 + 4 * g)
    wq, sw = _weights(1024, K, synth.seed_of(68, 1))
    _check(x.cuda(), wq, sw, "edge rows, one kernel")
    wq, sw = _weights(1024, K, synth.seed_of(68, 2), scale="pow2")
    _check(x.cuda(), wq, sw, "edge rows, one kernel, pow2", scale="pow2", accum="mx",
           outs=("bf16",))


def test_power_of_two_scales_both_accumulations():
    x = synth.act_bf16(64, 4096, seed=synth.seed_of(65, 0)).cuda()
    wq, sw = _weights(2048, 4096, synth.seed_of(65, 1), scale="pow2")
    _check(x, wq, sw, "pow2, fp8 slices", scale="pow2", accum="fp8", outs=("bf16",))
    _check(x, wq, sw, "pow2, matrix-core scales", scale="pow2", accum="mx", outs=("bf16",))
    _check(x, wq, sw, "pow2, default accumulation", scale="pow2")
    x = synth.act_bf16(5, 1024, seed=synth.seed_of(65, 2)).cuda()
    wq, sw = _weights(384, 1024, synth.seed_of(65, 3), scale="pow2")
    _check(x, wq, sw, "pow2, matrix-core scales, M=5", scale="pow2", accum="mx", outs=("bf16",))


@pytest.mark.parametrize("accum", ["fp8", "mx"])
def test_fp8_and_mx_refused_with_float32_output(accum):
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    sw = torch.ones((2, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(fq.Fp8rlError) as e:
        fq.gemm_fused_act(x, w, sw, out_dtype=torch.float32, accum=accum, scale="pow2")
    assert e.value.status == 7


def test_f16_slices_float32_output():
    x = synth.act_bf16(48, 4096, seed=synth.seed_of(66, 0)).cuda()
    _check(x, *_weights(1024, 4096, synth.seed_of(66, 1)), "f16 slices", outs=("f32",),
           accum="f16")


def test_workspace_reuse_determinism_and_canary():
    shapes = [(64, 4096, 4096), (20, 1024, 12288), (300, 768, 2048), (64, 4096, 4096),
              (1, 256, 2048), (65, 512, 1024)]
    need = max(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM_FUSED_ACT, *s) for s in shapes)
    ws = fq.new_workspace(need, "cuda")
    ws[fq.WORKSPACE_HEADER_BYTES:].fill_(0xC3)
    for i, (M, N, K) in enumerate(shapes):
        x = synth.act_bf16(M, K, seed=synth.seed_of(67, i)).cuda()
        wq, sw = _weights(N, K, synth.seed_of(67, 10 + i))
        dwq, dsw = to_dev_u8(wq), to_dev_f32(sw)
        ybuf = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device="cuda")
        fq.gemm_fused_act(x, dwq, dsw, y=ybuf[:, :N], workspace=ws)
        again = fq.gemm_fused_act(x, dwq, dsw, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ybuf[:, N:] == 7.0)
        assert torch.equal(ybuf[:, :N], again), (M, N, K)
        xq, sa = oq.quant_act_tok128(bits16(x))
        ref64 = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
        ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
        assert_gemm_close(gemm_out_to_f64(again), ref, ref64, "bf16", f"reuse {M}x{N}x{K}")
    assert int(ws[:fq.WORKSPACE_HEADER_BYTES].count_nonzero()) == 0


def test_zero_rows_and_rejected_shapes():
    w = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    sw = torch.ones((2, 2), dtype=torch.float32, device="cuda")
    y = fq.gemm_fused_act(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), w, sw)
    assert y.shape == (0, 256)
    with pytest.raises(fq.Fp8rlError):  # N not a multiple of 128 (host check)
        fq.gemm_fused_act(torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda"),
                          torch.zeros((200, 256), dtype=torch.uint8, device="cuda"), sw)
