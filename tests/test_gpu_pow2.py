"""GPU parity of the power-of-two scale option and the matrix-core-scaled GEMM (accum 'mx').

Quantizers: codes and scales bit-exact against the oracle's power-of-two rule (reading Q13 of
oracle/quant.py). GEMM with accum='mx': the E8M0 block scales are applied by the block-scaled FP8
matrix-core instruction, which also adds the running sum; each slice sum has the FP8 form's
precision, so it is offered for bf16 output only (checked against the contract tolerance on every
GEMM path: decode, mid-M fallback, large tiles, grouped). Float32 output of power-of-two operands
goes through the library's default (f16 slice sums) and is checked against the float32 contract.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import (assert_gemm_close, assert_within, bits16, fp8_slice_bound,
                            gemm_out_to_f64, to_dev_f32, to_dev_u8)
from tests.test_gpu_quant import _edge_weight
from workloads import synth

pytestmark = pytest.mark.gpu


def _check_weight_pow2(w, what):
    print(f"[quant_weight pow2] {what} {tuple(w.shape)}", flush=True)
    wq, sw = fq.quant_weight(w.cuda(), scale="pow2")
    torch.cuda.synchronize()
    rq, rs = oq.quant_weight_blk128(bits16(w), scale="pow2")
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), rs.view(np.uint32)), f"{what}: scales"
    assert int(np.count_nonzero(wq.cpu().numpy() != rq)) == 0, f"{what}: codes"


def _check_act_pow2(x, what):
    print(f"[quant_act pow2] {what} {tuple(x.shape)}", flush=True)
    xq, sa = fq.quant_act(x.cuda(), scale="pow2")
    torch.cuda.synchronize()
    rq, rs = oq.quant_act_tok128(bits16(x), scale="pow2")
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), rs.view(np.uint32)), f"{what}: scales"
    assert int(np.count_nonzero(xq.cpu().numpy() != rq)) == 0, f"{what}: codes"


def test_pow2_quantizers_tiny_and_edges():
    _check_weight_pow2(synth.weight_bf16(256, 256, seed=synth.seed_of(1, 0)), "tiny W")
    _check_act_pow2(synth.act_bf16(4, 256, seed=synth.seed_of(1, 1)), "tiny X")
    _check_weight_pow2(_edge_weight(), "edge blocks")
    _check_act_pow2(_edge_weight(), "edge blocks as rows")
    g = torch.Generator().manual_seed(5)
    w = (torch.randn((256, 512), generator=g) * 2.0 ** torch.randint(-40, 40, (256, 1),
                                                                     generator=g)).to(torch.bfloat16)
    _check_weight_pow2(w, "rows spread over 2^80")
    _check_act_pow2(w, "rows spread over 2^80 (activation)")


@pytest.mark.parametrize("idx", [0, 4, 6])
def test_pow2_qwen3_weights_full(idx):
    name, N, K = synth.DENSE_LINEARS_QWEN3_8B[idx]
    _check_weight_pow2(synth.weight_bf16(N, K, seed=synth.seed_of(2, idx), outlier_frac=0.001), name)


@pytest.mark.parametrize("M,K", [(64, 4096), (8192, 4096), (257, 1024)])
def test_pow2_activations(M, K):
    _check_act_pow2(synth.act_bf16(M, K, seed=synth.seed_of(3, M, K)), f"X[{M}][{K}]")


def test_pow2_batched_ex_matches_single():
    shapes = [(256, 384), (128, 128), (384, 256)]
    ws = [synth.weight_bf16(N, K, seed=900 + i).cuda() for i, (N, K) in enumerate(shapes)]
    wqs = [torch.empty(w.shape, dtype=torch.uint8, device="cuda") for w in ws]
    sws = [torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.float32,
                       device="cuda") for w in ws]
    fq.quant_weights(ws, wqs, sws, scale="pow2")
    for w, wq, sw in zip(ws, wqs, sws):
        a, b = fq.quant_weight(w, scale="pow2")
        torch.cuda.synchronize()
        assert torch.equal(a, wq) and torch.equal(b, sw)


def pow2_operands(M, N, K, seed):
    x = synth.act_bf16(M, K, seed=seed)
    w = synth.weight_bf16(N, K, seed=seed + 1, outlier_frac=0.001)
    xq, sa = oq.quant_act_tok128(bits16(x), scale="pow2")
    wq, sw = oq.quant_weight_blk128(bits16(w), scale="pow2")
    return xq, sa, wq, sw


def run_mx(xq, sa, wq, sw, what):
    M, N = xq.shape[0], wq.shape[0]
    print(f"[gemm mx] {what} M={M} N={N} K={xq.shape[1]}", flush=True)
    ref64 = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
    d = [to_dev_u8(xq), to_dev_f32(sa), to_dev_u8(wq), to_dev_f32(sw)]
    y = fq.gemm(*d, out_dtype=torch.bfloat16, accum="mx")
    torch.cuda.synchronize()
    ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
    wb = assert_gemm_close(gemm_out_to_f64(y), ref, ref64, "bf16", what)
    y = fq.gemm(*d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    wf = assert_gemm_close(gemm_out_to_f64(y), ref64.astype(np.float32).astype(np.float64), ref64,
                           "f32", what + " f32 (default accumulation)")
    print(f"    worst err/bound bf16 {wb:.3f} f32 {wf:.3f}", flush=True)


@pytest.mark.parametrize("M,N,K", [(4, 256, 256), (64, 4096, 4096), (64, 1024, 12288), (17, 512, 2048),
                                   (1, 256, 1024), (48, 2048, 1280), (40, 24576, 640),
                                   (9, 1536, 1152), (200, 512, 1024),
                                   (1024, 1024, 2048), (2048 + 37, 768, 1536), (8192, 4096, 4096)])
def test_mx_gemm_all_paths(M, N, K):
    run_mx(*pow2_operands(M, N, K, 7000 + M + N + K), f"{M}x{N}x{K}")


def test_mx_grouped_moe_and_ragged():
    counts = [0, 1, 130, 0, 5, 257, 0]
    E, N, K = len(counts), 256, 384
    M = sum(counts)
    x = synth.act_bf16(M, K, seed=81)
    xq, sa = oq.quant_act_tok128(bits16(x), scale="pow2")
    w = bits16(synth.weight_bf16(N, K, seed=82, batch=E))
    wq = np.empty((E, N, K), np.uint8)
    sw = np.empty((E, N // 128, K // 128), np.float32)
    for e in range(E):
        wq[e], sw[e] = oq.quant_weight_blk128(w[e], scale="pow2")
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    ref64 = og.grouped_gemm_blockscaled(xq, sa, wq, sw, off, out="f64")
    d = [to_dev_u8(xq), to_dev_f32(sa), to_dev_u8(wq), to_dev_f32(sw), torch.from_numpy(off).cuda()]
    y = fq.grouped_gemm(*d, out_dtype=torch.bfloat16, accum="mx")
    torch.cuda.synchronize()
    ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
    assert_gemm_close(gemm_out_to_f64(y), ref, ref64, "bf16", "grouped mx ragged")
    y = fq.grouped_gemm(*d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(gemm_out_to_f64(y), ref64.astype(np.float32).astype(np.float64), ref64,
                      "f32", "grouped pow2 f32 (default accumulation)")


def test_mx_and_fp8_accum_on_random_pow2_operands_derived_bound():
    """Stress test: random full-range codes with power-of-two scales spread over 2^24, through
    the FP32-rescale path (accum='fp8') and the matrix-core scaled path (bf16 output): both
    within the FP8 form's derived bound of the exact result."""
    rng = np.random.default_rng(91)
    M, N, K = 64, 2048, 4096
    xq = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    wq = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x7E
    wq[(wq & 0x7F) == 0x7F] = 0xFE
    sa = (2.0 ** rng.integers(-20, 4, size=(M, K // 128))).astype(np.float32)
    sw = (2.0 ** rng.integers(-20, 4, size=(N // 128, K // 128))).astype(np.float32)
    ref64 = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
    d = [to_dev_u8(xq), to_dev_f32(sa), to_dev_u8(wq), to_dev_f32(sw)]
    a = gemm_out_to_f64(fq.gemm(*d, out_dtype=torch.bfloat16, accum="fp8"))
    b = gemm_out_to_f64(fq.gemm(*d, out_dtype=torch.bfloat16, accum="mx"))
    bound = fp8_slice_bound(xq, sa, wq, sw) + 2.0 ** -8 * np.abs(ref64)
    assert_within(a, ref64, bound, "fp8 accum")
    assert_within(b, ref64, bound, "mx accum")


@pytest.mark.parametrize("M,N,K", [(64, 4096, 4096), (1024, 6144, 4096)])
def test_gpu_scale_formats_against_unquantized_product(M, N, K):
    """The GPU's two scale formats end to end (quantizers and GEMM on the GPU: FP32 scales with
    FP8 slice sums, power-of-two scales with the matrix-core-scaled GEMM, bf16 output) against
    the exact product of the unquantized bf16 operands: both within the E4M3 bound, and the
    power-of-two form's relative error 1-2x the FP32 form's, as the oracle's comparison finds."""
    x = synth.act_bf16(M, K, seed=synth.seed_of(71, M, K))
    w = synth.weight_bf16(N, K, seed=synth.seed_of(71, N, K), outlier_frac=0.001)
    ref = x.double() @ w.double().t()
    rel = {}
    for scale, accum in (("fp32", None), ("pow2", "mx")):
        xq, sa = fq.quant_act(x.cuda(), scale=scale)
        wq, sw = fq.quant_weight(w.cuda(), scale=scale)
        y = fq.gemm(xq, sa, wq, sw, accum=accum)
        torch.cuda.synchronize()
        rel[scale] = float(torch.linalg.norm(y.double().cpu() - ref) / torch.linalg.norm(ref))
    print(f"[scale formats] {M}x{N}x{K}: relative error fp32 {rel['fp32']:.3e}, "
          f"pow2 {rel['pow2']:.3e}, ratio {rel['pow2'] / rel['fp32']:.3f}", flush=True)
    assert rel["fp32"] < 2.0 ** -4 and rel["pow2"] < 2.0 ** -4
    assert 0.95 < rel["pow2"] / rel["fp32"] < 2.0
