"""GPU parity at the workloads' full sizes, in the launch configurations the benchmark times.

* Llama-3.1-8B weight sync: all 224 linear weights of 32 layers (6.98e9 elements) re-quantized by
  the batched entry point in 7 launches of 32 matrices, exactly as the benchmark runs it. Layers
  0, 15 and 31 are checked whole against the oracle; every other matrix on three sampled 128x128
  blocks (first, last and a seeded one). Codes and scales bit-exact.
* Qwen3-30B-A3B expert weights (128 experts, gate/up [1536][2048] and down [2048][768]) re-quantized
  as the benchmark does it: each [E][N][K] tensor as one [E*N][K] matrix (its 128x128 blocks never
  straddle experts), both in one batched launch; six experts of each checked whole against the
  oracle run on that expert alone.
* The decoder-block GEMMs in the serving layout (q/k/v and gate/up weights concatenated along N):
  Qwen3-8B decode (M = 64) checked whole, Qwen3-8B prefill (M = 8192) and the Llama-3.1-8B MLP
  (M = 256 whole, M = 4096 on sampled rows). Operands are quantized by the oracle from the seeded
  synthetic tensors; the GEMM runs through the same entry point and planner as the benchmark.
  Sampled rows: GEMM rows are independent, so the oracle computes just those rows of the product;
  rms(ref) in the bf16 tolerance is taken over the sampled rows.
* The FP8 backward of the Qwen3-8B gate/up linear over 8192 tokens as the benchmark runs it: the
  three quantizers bit-exact at full size, Dgrad (K = 24576) and Wgrad (contraction over the 8192
  tokens, the default f16 slice sums) on sampled output rows, both within the bf16 tolerance.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import backward as ob
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import (assert_gemm_close, bits16,
                            gemm_out_to_f64, to_dev_f32, to_dev_u8)
from workloads import synth

pytestmark = pytest.mark.gpu


def test_llama31_8b_weight_sync_32_layers():
    layers = 32
    shapes = [(N, K) for _ in range(layers) for _, N, K in synth.LLAMA31_8B_LAYER_LINEARS]
    per_layer = len(synth.LLAMA31_8B_LAYER_LINEARS)
    print(f"[weight sync] {len(shapes)} matrices, "
          f"{sum(N * K for N, K in shapes)} elements", flush=True)
    ws, wqs, sws = [], [], []
    for i, (N, K) in enumerate(shapes):
        ws.append(synth.weight_bf16(N, K, seed=3000 + i, outlier_frac=0.001, device="cuda"))
        wqs.append(torch.empty((N, K), dtype=torch.uint8, device="cuda"))
        sws.append(torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda"))
    descs = fq.weight_descs(ws, wqs, sws)
    fq.quant_weights(None, None, None, descs=descs)  # 224 matrices -> 7 launches of 32
    torch.cuda.synchronize()

    full_layers = (0, 15, 31)
    rng = np.random.default_rng(4321)
    for i, (N, K) in enumerate(shapes):
        layer = i // per_layer
        if layer in full_layers:
            rq, rs = oq.quant_weight_blk128(bits16(ws[i]))
            assert np.array_equal(sws[i].cpu().numpy().view(np.uint32), rs.view(np.uint32)), i
            bad = int(np.count_nonzero(wqs[i].cpu().numpy() != rq))
            assert bad == 0, f"matrix {i} ({N}x{K}): {bad} codes differ"
            continue
        nb, kb = N // 128, K // 128
        for bi, bj in ((0, 0), (nb - 1, kb - 1), (int(rng.integers(nb)), int(rng.integers(kb)))):
            rows, cols = slice(128 * bi, 128 * bi + 128), slice(128 * bj, 128 * bj + 128)
            rq, rs = oq.quant_weight_blk128(bits16(ws[i][rows, cols]))
            got_s = sws[i][bi, bj].reshape(1, 1).cpu().numpy()
            assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32)), (i, bi, bj)
            assert np.array_equal(wqs[i][rows, cols].cpu().numpy(), rq), (i, bi, bj)
    print("    layers 0, 15, 31 whole; 3 blocks of every other matrix", flush=True)


def test_qwen3_30b_a3b_expert_requant_one_launch():
    E, H, I = 128, 2048, 768
    print(f"[expert requant] E={E} gate/up [{2 * I}][{H}], down [{H}][{I}]", flush=True)
    w1 = synth.weight_bf16(2 * I, H, seed=43, batch=E, device="cuda")
    w2 = synth.weight_bf16(H, I, seed=44, batch=E, device="cuda")
    wq1 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device="cuda")
    sw1 = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device="cuda")
    wq2 = torch.empty((E, H, I), dtype=torch.uint8, device="cuda")
    sw2 = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device="cuda")
    fq.quant_weights([w1.view(E * 2 * I, H), w2.view(E * H, I)],
                     [wq1.view(E * 2 * I, H), wq2.view(E * H, I)],
                     [sw1.view(E * 2 * I // 128, H // 128), sw2.view(E * H // 128, I // 128)])
    torch.cuda.synchronize()
    for w, wq, sw in ((w1, wq1, sw1), (w2, wq2, sw2)):
        for e in (0, 1, 63, 64, 100, 127):
            rq, rs = oq.quant_weight_blk128(bits16(w[e]))
            assert np.array_equal(sw[e].cpu().numpy().view(np.uint32), rs.view(np.uint32)), e
            assert np.array_equal(wq[e].cpu().numpy(), rq), e


def _operands(M, N, K, seed):
    x = synth.act_bf16(M, K, seed=seed)
    w = synth.weight_bf16(N, K, seed=seed + 1, outlier_frac=0.001)
    xq, sa = oq.quant_act_tok128(bits16(x))
    wq, sw = oq.quant_weight_blk128(bits16(w))
    return xq, sa, wq, sw


def _sample_rows(M, n_random, seed):
    fixed = {0, 1, 2, 3, 15, 16, 63, 64, 127, 128, 255, 256, M // 2 - 1, M // 2, M - 2, M - 1}
    rng = np.random.default_rng(seed)
    rows = fixed | set(int(r) for r in rng.choice(M, size=n_random, replace=False))
    return np.array(sorted(r for r in rows if 0 <= r < M))


def _check_gemm(M, N, K, seed, rows=None, what=""):
    print(f"[gemm full size] {what} M={M} N={N} K={K} "
          f"rows={'all' if rows is None else len(rows)}", flush=True)
    xq, sa, wq, sw = _operands(M, N, K, seed)
    y = fq.gemm(to_dev_u8(xq), to_dev_f32(sa), to_dev_u8(wq), to_dev_f32(sw),
                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = gemm_out_to_f64(y)
    if rows is not None:
        got = got[rows]
        xq, sa = xq[rows], sa[rows]
    ref64 = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
    ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
    worst = assert_gemm_close(got, ref, ref64, "bf16", what)
    print(f"    worst err/bound {worst:.3f}", flush=True)


# serving layout: q/k/v concatenated (6144 rows), gate/up concatenated
QWEN3_GEMMS = (("qkv_proj", 6144, 4096), ("o_proj", 4096, 4096), ("gate_up_proj", 24576, 4096),
               ("down_proj", 4096, 12288))
LLAMA_MLP_GEMMS = (("gate_up_proj", 28672, 4096), ("down_proj", 4096, 14336))


@pytest.mark.parametrize("idx", range(len(QWEN3_GEMMS)))
def test_qwen3_8b_decode_gemms_whole(idx):
    name, N, K = QWEN3_GEMMS[idx]
    _check_gemm(64, N, K, 5100 + idx, what=f"qwen3-8b decode {name}")


@pytest.mark.parametrize("idx", (0, 2, 3))  # q_proj at M = 8192 is checked whole in test_gpu_gemm
def test_qwen3_8b_prefill_gemms_sampled_rows(idx):
    name, N, K = QWEN3_GEMMS[idx]
    _check_gemm(8192, N, K, 5200 + idx, rows=_sample_rows(8192, 48, 5250 + idx),
                what=f"qwen3-8b prefill {name}")


@pytest.mark.parametrize("idx", range(len(LLAMA_MLP_GEMMS)))
def test_llama31_8b_mlp_m256_whole(idx):
    name, N, K = LLAMA_MLP_GEMMS[idx]
    _check_gemm(256, N, K, 5300 + idx, what=f"llama-3.1-8b mlp M=256 {name}")


@pytest.mark.parametrize("idx", range(len(LLAMA_MLP_GEMMS)))
def test_llama31_8b_mlp_m4096_sampled_rows(idx):
    name, N, K = LLAMA_MLP_GEMMS[idx]
    _check_gemm(4096, N, K, 5400 + idx, rows=_sample_rows(4096, 48, 5450 + idx),
                what=f"llama-3.1-8b mlp M=4096 {name}")


def test_qwen3_8b_gate_up_backward_8192_tokens():
    T, N, K = 8192, 24576, 4096
    print(f"[backward full size] gate/up {N}x{K} over {T} tokens", flush=True)
    dy = synth.act_bf16(T, N, seed=synth.seed_of(46, 0)) * 0.01
    x = synth.act_bf16(T, K, seed=synth.seed_of(46, 1))
    w = synth.weight_bf16(N, K, seed=synth.seed_of(46, 2), outlier_frac=0.001)
    dyt, s_dyt, dyq, s_dy = fq.quant_colwise(dy.cuda(), rowwise=True)
    xt, s_xt, _, _ = fq.quant_colwise(x.cuda())
    wqt, swt, _, _ = fq.quant_weight_t(w.cuda())
    dx = fq.gemm(dyq, s_dy, wqt, swt)  # Dgrad: [T][K], contraction over N
    dw = fq.gemm_rowscaled(dyt, s_dyt, xt, s_xt)  # Wgrad: [N][K], contraction over T
    torch.cuda.synchronize()

    def same(got, ref, what):
        got = got.cpu().numpy()
        if got.dtype == np.float32:
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), what
        else:
            assert int(np.count_nonzero(got != ref)) == 0, what

    r_dyq, r_sdy = oq.quant_act_tok128(bits16(dy))
    same(dyq, r_dyq, "dY codes (1x128)")
    same(s_dy, r_sdy, "dY scales (1x128)")
    r_dyt, r_sdyt = ob.quant_colwise128(bits16(dy))
    same(dyt, r_dyt, "dY codes (128x1, transposed)")
    same(s_dyt, r_sdyt, "dY scales (128x1)")
    r_xt, r_sxt = ob.quant_colwise128(bits16(x))
    same(xt, r_xt, "X codes (128x1, transposed)")
    same(s_xt, r_sxt, "X scales (128x1)")
    r_wqt, r_swt = ob.quant_weight_blk128_t(bits16(w))
    same(wqt, r_wqt, "W^T codes")
    same(swt, r_swt, "W^T scales")

    rows = _sample_rows(T, 48, 5500)
    ref64 = og.gemm_blockscaled(r_dyq[rows], r_sdy[rows], r_wqt, r_swt, out="f64")
    ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
    got = gemm_out_to_f64(dx[torch.from_numpy(rows).cuda()])
    print(f"    dX worst err/bound {assert_gemm_close(got, ref, ref64, 'bf16', 'dX'):.3f}", flush=True)

    rows_w = _sample_rows(N, 48, 5501)
    ref64w = ob.gemm_rowscaled(r_dyt[rows_w], r_sdyt[rows_w], r_xt, r_sxt, out="f64")
    refw = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64w))
    got_w = gemm_out_to_f64(dw[torch.from_numpy(rows_w).cuda()])
    print(f"    dW worst err/bound {assert_gemm_close(got_w, refw, ref64w, 'bf16', 'dW'):.3f}",
          flush=True)
