"""GPU parity of the grouped GEMM on bf16 activations (fp8rl_grouped_gemm_w8a8_fused_act_quant).

Grouped row r multiplies token row row_ids[r] (clamped to the token range), quantized in 1x128
groups, with its expert's weights. Two checks on every case:

* against the oracle: the oracle's 1x128 quantization of the tokens, its rows taken in row_ids
  order, through the oracle's grouped GEMM, within the GEMM contract (|gpu - ref| <= 2^-7 |ref| +
  1e-3 rms(ref) for bf16 output, <= 1e-5 rms(ref) for float32 output);
* bit-identical to the library's unfused path on the gathered bf16 rows: fp8rl_quant_act_tok128
  on x[row_ids] followed by fp8rl_grouped_gemm_w8a8 (a 1x128 group lies within one row, so
  quantizing a token once gives the codes of every copy of it).

Inputs: seeded synthetic tokens (N(0, 1) with outlier channels), one synthetic weight tensor per
expert, and the Zipf(1.1) top-8 router of the Qwen3-30B-A3B layer (4096 tokens, 128 experts) or
small ragged routings with empty and single-row experts.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import assert_gemm_close, bits16, gemm_out_to_f64, to_dev_f32, to_dev_u8
from workloads import synth

pytestmark = pytest.mark.gpu


def _experts(E, N, K, seed, scale="fp32"):
    w = bits16(synth.weight_bf16(N, K, seed=seed, batch=E))
    wq = np.empty((E, N, K), np.uint8)
    sw = np.empty((E, N // 128, K // 128), np.float32)
    for e in range(E):
        wq[e], sw[e] = oq.quant_weight_blk128(w[e], scale=scale)
    return wq, sw


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


def _check(x, row_ids, wq, sw, off, what, scale="fp32", outs=("bf16", "f32"), accum=None,
           oracle=True):
    """x: bf16 tokens on the GPU; row_ids: int32 numpy array (or None: grouped rows = x's rows);
    wq / sw: oracle codes and scales [E][N][K]; off: expert offsets."""
    T, K = x.shape
    M = T if row_ids is None else row_ids.size
    E, N = wq.shape[0], wq.shape[1]
    print(f"[grouped fused act] {what} tokens={T} M_total={M} E={E} N={N} K={K} scale={scale} "
          f"accum={accum}", flush=True)
    src = np.arange(T) if row_ids is None else np.clip(row_ids.astype(np.int64), 0, T - 1)
    d_ids = None if row_ids is None else torch.from_numpy(row_ids).cuda()
    d_off = torch.from_numpy(off).cuda()
    dwq, dsw = to_dev_u8(wq), to_dev_f32(sw)
    if oracle:
        xq, sa = oq.quant_act_tok128(bits16(x), scale=scale)
        ref64 = og.grouped_gemm_blockscaled(xq[src], sa[src], wq, sw, off, out="f64")
    x_gathered = x[torch.from_numpy(src).cuda()]
    for out in outs:
        dt = torch.bfloat16 if out == "bf16" else torch.float32
        y = fq.grouped_gemm_fused_act(x, dwq, dsw, d_off, row_ids=d_ids, out_dtype=dt,
                                      accum=accum, scale=scale)
        gxq, gsa = fq.quant_act(x_gathered, scale=scale)
        y2 = fq.grouped_gemm(gxq, gsa, dwq, dsw, d_off, out_dtype=dt, accum=accum)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"{what} {out}: differs from quant_act + grouped GEMM"
        if oracle:
            ref = (og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64)) if out == "bf16"
                   else ref64.astype(np.float32).astype(np.float64))
            w = assert_gemm_close(gemm_out_to_f64(y), ref, ref64, out, what)
            print(f"    {out}: worst err/bound {w:.3f}", flush=True)


def test_moe_gate_up_full_size_token_gather():
    """Qwen3-30B-A3B gate/up (2048 -> 1536): the 4096 tokens quantized once, 32768 grouped rows
    read through the router's token indices, 128 distinct experts."""
    counts, ids = synth.moe_routing(4096, 128, 8, seed=synth.seed_of(5, 0))
    x = synth.act_bf16(4096, 2048, seed=5100, device="cuda")
    wq, sw = _experts(128, 1536, 2048, 5101)
    _check(x, ids.numpy(), wq, sw, _offsets(counts.numpy()), "moe gate_up gather",
           outs=("bf16",))


def test_moe_down_full_size_grouped_input():
    """Qwen3-30B-A3B down (768 -> 2048): the input is already in expert order (no row ids)."""
    counts = synth.moe_routing_counts(4096, 128, 8, seed=synth.seed_of(5, 0))
    x = synth.act_bf16(int(counts.sum()), 768, seed=5102, device="cuda")
    wq, sw = _experts(128, 2048, 768, 5103)
    _check(x, None, wq, sw, _offsets(counts.numpy()), "moe down", outs=("bf16",))


def test_float32_output_and_mx_on_a_routing_subset():
    counts, ids = synth.moe_routing(512, 16, 4, seed=5104)
    x = synth.act_bf16(512, 1024, seed=5105, device="cuda")
    off = _offsets(counts.numpy())
    wq, sw = _experts(16, 512, 1024, 5106)
    _check(x, ids.numpy(), wq, sw, off, "routed subset")
    wq2, sw2 = _experts(16, 512, 1024, 5106, scale="pow2")
    _check(x, ids.numpy(), wq2, sw2, off, "routed subset (mx)", scale="pow2", outs=("bf16",),
           accum="mx")


def test_ragged_experts_duplicates_and_clamped_ids():
    """Empty, single-row and multi-tile experts; a token sent to one expert several times; ids
    below 0 and past the last token read the first / last token."""
    counts = [0, 1, 130, 0, 5, 257, 0, 3]
    M = int(sum(counts))
    rng = np.random.default_rng(5107)
    T = 97
    ids = rng.integers(0, T, size=M).astype(np.int32)
    ids[:4] = [-5, T, T + 1000, -(2 ** 31)]
    ids[10:14] = 42
    x = synth.act_bf16(T, 384, seed=5108, device="cuda")
    wq, sw = _experts(len(counts), 256, 384, 5109)
    _check(x, ids, wq, sw, _offsets(counts), "ragged, duplicates, clamped ids")


def test_token_rows_with_a_row_pitch():
    """Tokens taken from a wider buffer (row pitch above K)."""
    counts, ids = synth.moe_routing(300, 8, 2, seed=5110)
    buf = synth.act_bf16(300, 1024 + 256, seed=5111, device="cuda")
    x = buf[:, 128:1152]
    wq, sw = _experts(8, 384, 1024, 5112)
    _check(x, ids.numpy(), wq, sw, _offsets(counts.numpy()), "pitched tokens")


def test_k_beyond_dma_tiles_gathers_codes_first():
    """K = 32896 (257 slices): the grouped GEMM's register-staged tiles, fed by a gather of the
    token codes into the workspace."""
    counts = [3, 0, 70, 130]
    rng = np.random.default_rng(5113)
    ids = rng.integers(0, 50, size=sum(counts)).astype(np.int32)
    x = synth.act_bf16(50, 32896, seed=5114, device="cuda")
    wq, sw = _experts(4, 256, 32896, 5115)
    _check(x, ids, wq, sw, _offsets(counts), "K=32896 gather")


def test_workspace_header_untouched_and_shared_with_dense_gemm():
    """The call writes nothing into the workspace's counter header, so one workspace serves it
    and the dense split-K GEMM (which needs those counters zero) in any order; and it gives the
    same bits every call."""
    counts, ids = synth.moe_routing(256, 8, 2, seed=5116)
    x = synth.act_bf16(256, 1024, seed=5117, device="cuda")
    wq, sw = _experts(8, 512, 1024, 5118)
    dwq, dsw = to_dev_u8(wq), to_dev_f32(sw)
    d_off = torch.from_numpy(_offsets(counts.numpy())).cuda()
    d_ids = ids.cuda()
    dense_shape = (64, 4096, 4096)  # the split-K decode GEMM
    need = max(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GROUPED_GEMM_FUSED_ACT, 512, 512, 1024, 8),
               fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, *dense_shape))
    assert fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, *dense_shape) > 0
    ws = fq.new_workspace(need, "cuda")
    hdr = fq.WORKSPACE_HEADER_BYTES
    xd = synth.act_bf16(64, 4096, seed=5119, device="cuda")
    wd = synth.weight_bf16(4096, 4096, seed=5120, device="cuda")
    xdq, sdq = fq.quant_act(xd)
    wdq, swd = fq.quant_weight(wd)
    y_dense_ref = fq.gemm(xdq, sdq, wdq, swd)
    ys = []
    for _ in range(2):
        ys.append(fq.grouped_gemm_fused_act(x, dwq, dsw, d_off, row_ids=d_ids, workspace=ws))
        torch.cuda.synchronize()
        assert int(ws[:hdr].view(torch.uint8).count_nonzero()) == 0
        y_dense = fq.gemm(xdq, sdq, wdq, swd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_dense, y_dense_ref)
    assert torch.equal(ys[0], ys[1])
