"""GPU parity of the FP8 backward pass (Dgrad and Wgrad operands and products) against the oracle.

Quantized codes and scales must be bit-exact: the transposed weight copy (and the row-major codes
from the same read), the 128x1 token-group quantization stored transposed (and the 1x128 row
quantization from the same read). The row-scaled GEMM is held to the GEMM contract of the forward
tests on every kernel path its planner can pick (small tiles, large tiles, split K, the DMA-fed
large-M tiles), with FP8, f16 and matrix-core-scaled slice sums. Inputs: Qwen3-8B-shaped weights
and N(0, 1) activations / gradients with outlier channels, seeded.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import backward as ob
from oracle import quant as oq
from tests.gpu_util import assert_gemm_close, assert_within, bits16, fp8_slice_bound, gemm_out_to_f64
from workloads import synth

pytestmark = pytest.mark.gpu


def _u32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("N,K,scale", [(4096, 4096, "fp32"), (1024, 4096, "fp32"), (4096, 12288, "fp32"),
                                       (384, 640, "fp32"), (4096, 4096, "pow2")])
def test_weight_transposed_copy(N, K, scale):
    w = synth.weight_bf16(N, K, seed=synth.seed_of(40, N, K), outlier_frac=0.001)
    print(f"[quant_weight_t] {N}x{K} {scale}", flush=True)
    wqt, swt, wq, sw = fq.quant_weight_t(w.cuda(), rowmajor=True, scale=scale)
    torch.cuda.synchronize()
    rqt, rst = ob.quant_weight_blk128_t(bits16(w), scale=scale)
    rq, rs = oq.quant_weight_blk128(bits16(w), scale=scale)
    assert np.array_equal(_u32(swt.cpu().numpy()), _u32(rst))
    assert np.array_equal(_u32(sw.cpu().numpy()), _u32(rs))
    assert int(np.count_nonzero(wqt.cpu().numpy() != rqt)) == 0
    assert int(np.count_nonzero(wq.cpu().numpy() != rq)) == 0


def test_weight_transposed_only_with_pitch():
    N, K = 512, 768
    w = synth.weight_bf16(N, 2 * K, seed=synth.seed_of(41, 0))[:, :K].cuda()  # row pitch 2K
    wqt = torch.full((K, N + 64), 0xA5, dtype=torch.uint8, device="cuda")
    swt = torch.empty((K // 128, N // 128), dtype=torch.float32, device="cuda")
    fq.quant_weight_t(w, wqt=wqt[:, :N], swt=swt)
    torch.cuda.synchronize()
    rqt, rst = ob.quant_weight_blk128_t(bits16(w))
    got = wqt.cpu().numpy()
    assert np.array_equal(got[:, :N], rqt) and np.all(got[:, N:] == 0xA5)
    assert np.array_equal(_u32(swt.cpu().numpy()), _u32(rst))


@pytest.mark.parametrize("M,K,scale", [(128, 128, "fp32"), (256, 4096, "fp32"), (8192, 4096, "fp32"),
                                       (4096, 12288, "fp32"), (1024, 1024, "pow2")])
def test_colwise_and_rowwise_from_one_read(M, K, scale):
    x = synth.act_bf16(M, K, seed=synth.seed_of(42, M, K))
    print(f"[quant_colwise] {M}x{K} {scale}", flush=True)
    xtq, sat, xq, sa = fq.quant_colwise(x.cuda(), rowwise=True, scale=scale)
    torch.cuda.synchronize()
    rtq, rst = ob.quant_colwise128(bits16(x), scale=scale)
    rq, rs = oq.quant_act_tok128(bits16(x), scale=scale)
    assert np.array_equal(_u32(sat.cpu().numpy()), _u32(rst))
    assert int(np.count_nonzero(xtq.cpu().numpy() != rtq)) == 0
    assert np.array_equal(_u32(sa.cpu().numpy()), _u32(rs))
    assert int(np.count_nonzero(xq.cpu().numpy() != rq)) == 0


def test_colwise_edge_columns():
    # columns that are all zero, a single outlier, negatives, bf16 subnormals and huge values
    M, K = 256, 256
    x = synth.act_bf16(M, K, seed=synth.seed_of(43, 0)).clone()
    x[:, 0] = 0.0
    x[:, 1] = 0.0
    x[77, 1] = -3.0
    x[:, 2] = -torch.arange(1, M + 1, dtype=torch.float32).to(torch.bfloat16)
    x[:, 3] = torch.tensor(2.0 ** -130).to(torch.bfloat16)
    x[:128, 4] = 3.0e38
    x[:, 5] = -0.0
    xtq, sat, _, _ = fq.quant_colwise(x.cuda())
    torch.cuda.synchronize()
    rtq, rst = ob.quant_colwise128(bits16(x))
    assert np.array_equal(_u32(sat.cpu().numpy()), _u32(rst))
    assert np.array_equal(xtq.cpu().numpy(), rtq)


def _rowscaled_operands(M, N, K, seed, pow2=False):
    """Wgrad-like operands: 1x128-quantized rows of gradient- and activation-shaped tensors."""
    a = synth.act_bf16(M, K, seed=synth.seed_of(44, seed, 0))
    b = synth.act_bf16(N, K, seed=synth.seed_of(44, seed, 1))
    scale = "pow2" if pow2 else "fp32"
    aq, sa = oq.quant_act_tok128(bits16(a), scale=scale)
    bq, sb = oq.quant_act_tok128(bits16(b), scale=scale)
    return aq, sa, bq, sb


def _check_rowscaled(M, N, K, out, accum, seed=0, pow2=False):
    aq, sa, bq, sb = _rowscaled_operands(M, N, K, seed, pow2)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    print(f"[gemm_rowscaled] {M}x{N}x{K} out={out} accum={accum}", flush=True)
    y = fq.gemm_rowscaled(t(aq), t(sa), t(bq), t(sb), out_dtype=dt, accum=accum)
    torch.cuda.synchronize()
    got = gemm_out_to_f64(y)
    ref64 = ob.gemm_rowscaled(aq, sa, bq, sb, out="f64")
    if out == "bf16":
        ref = oq_bf16(ob.gemm_rowscaled(aq, sa, bq, sb, out="bf16"))
        return assert_gemm_close(got, ref, ref64, "bf16", f"{M}x{N}x{K}")
    return assert_gemm_close(got, ref64.astype(np.float32).astype(np.float64), ref64, "f32",
                             f"{M}x{N}x{K}")


def oq_bf16(bits):
    from oracle import gemm as og
    return og.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (64, 1024, 1024), (200, 384, 512), (640, 512, 1024),
                                   (1024, 1024, 2048), (4096, 4096, 1024), (1100, 640, 640),
                                   (300, 16384, 512)])
@pytest.mark.parametrize("accum", [None, "fp8", "mx"])
def test_rowscaled_gemm_bf16(M, N, K, accum):
    _check_rowscaled(M, N, K, "bf16", accum, pow2=accum == "mx")


@pytest.mark.parametrize("M,N,K", [(64, 256, 512), (512, 512, 512), (1024, 512, 1024),
                                   (4096, 1024, 2048), (300, 16384, 512)])
@pytest.mark.parametrize("accum", [None, "f16"])
def test_rowscaled_gemm_f32(M, N, K, accum):
    _check_rowscaled(M, N, K, "f32", accum, seed=1)


@pytest.mark.parametrize("accum", ["fp8", "mx"])
def test_rowscaled_fp8_and_mx_refused_with_float32_output(accum):
    aq, sa, bq, sb = _rowscaled_operands(64, 256, 512, 2, accum == "mx")
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    with pytest.raises(fq.Fp8rlError) as e:
        fq.gemm_rowscaled(t(aq), t(sa), t(bq), t(sb), out_dtype=torch.float32, accum=accum)
    assert e.value.status == 7  # FP8RL_ERR_ARG


@pytest.mark.parametrize("M,N,K", [(256, 512, 1024), (1024, 384, 2048)])
def test_rowscaled_fp8_slices_random_operands_derived_bound(M, N, K):
    """Stress test of the opt-in FP8 slice sums of the row-scaled GEMM (bf16 output): random
    full-range codes with scales spread over 2^24, against the FP8 form's derived bound."""
    rng = np.random.default_rng(4400 + M)
    aq = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    bq = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x7E
    bq[(bq & 0x7F) == 0x7F] = 0xFE
    sa = (2.0 ** rng.uniform(-20, 4, size=(M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.uniform(-20, 4, size=(N, K // 128))).astype(np.float32)
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    y = fq.gemm_rowscaled(t(aq), t(sa), t(bq), t(sb), out_dtype=torch.bfloat16, accum="fp8")
    torch.cuda.synchronize()
    ref64 = ob.gemm_rowscaled(aq, sa, bq, sb, out="f64")
    bound = fp8_slice_bound(aq, sa, bq, sb, b_rows=True) + 2.0 ** -8 * np.abs(ref64)
    assert_within(gemm_out_to_f64(y), ref64, bound, f"rowscaled fp8 slices {M}x{N}x{K}")


def test_linear_backward_end_to_end():
    # dX and dW of a Qwen3-8B o_proj-shaped linear (4096x4096) over 1024 tokens, every step on the
    # GPU through the C ABI, against the oracle's FP8 backward
    M, N, K = 1024, 4096, 4096
    dy = synth.act_bf16(M, N, seed=synth.seed_of(45, 0)) * 0.01
    x = synth.act_bf16(M, K, seed=synth.seed_of(45, 1))
    w = synth.weight_bf16(N, K, seed=synth.seed_of(45, 2), outlier_frac=0.001)
    print("[linear backward] 1024 tokens, 4096x4096", flush=True)
    dyt, s_dyt, dyq, s_dy = fq.quant_colwise(dy.cuda(), rowwise=True)
    xt, s_xt, _, _ = fq.quant_colwise(x.cuda())
    wqt, swt, _, _ = fq.quant_weight_t(w.cuda())
    dx = fq.gemm(dyq, s_dy, wqt, swt)
    dw = fq.gemm_rowscaled(dyt, s_dyt, xt, s_xt)  # the library's default form (f16 slice sums)
    torch.cuda.synchronize()
    rdx, rdw = ob.linear_backward_fp8(bits16(dy), bits16(x), bits16(w), out="f64")
    rdx_b, rdw_b = ob.linear_backward_fp8(bits16(dy), bits16(x), bits16(w), out="bf16")
    assert_gemm_close(gemm_out_to_f64(dx), oq_bf16(rdx_b), rdx, "bf16", "dX")
    # Wgrad sums over the tokens, where activation outlier channels make single slices large
    # against the result; the default form's float32-grade slice sums keep the bf16 contract.
    # (A float32 dW is not held to 1e-5 rms here: where outlier rows of dY meet outlier columns
    # of X an element is ~256x the rms, and one float32 ulp there already exceeds that bound.)
    assert_gemm_close(gemm_out_to_f64(dw), oq_bf16(rdw_b), rdw, "bf16", "dW")
