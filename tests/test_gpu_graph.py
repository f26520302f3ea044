"""Graph capture of the hot path (as the benchmark replays it): every replay must equal the
eager result, with eager work and synchronizations between replays."""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import assert_gemm_close, bits16
from workloads import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_and_oracle():
    M = 64
    shapes = [(1024, 4096), (4096, 4096), (4096, 12288)]  # split-K and plain GEMM launches
    ws = [synth.weight_bf16(N, K, seed=600 + i, outlier_frac=0.001).cuda()
          for i, (N, K) in enumerate(shapes)]
    xs = [synth.act_bf16(M, K, seed=610 + i).cuda() for i, (N, K) in enumerate(shapes)]
    wqs = [torch.empty(w.shape, dtype=torch.uint8, device="cuda") for w in ws]
    sws = [torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.float32,
                       device="cuda") for w in ws]
    xqs = [torch.empty(x.shape, dtype=torch.uint8, device="cuda") for x in xs]
    sas = [torch.empty((M, x.shape[1] // 128), dtype=torch.float32, device="cuda") for x in xs]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N, K in shapes]
    wss = [fq.new_workspace(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, M, N, K), "cuda")
           for N, K in shapes]
    descs = fq.weight_descs(ws, wqs, sws)

    def step():
        fq.quant_weights(None, None, None, descs=descs)
        for i in range(len(shapes)):
            fq.quant_act(xs[i], xqs[i], sas[i])
            fq.gemm(xqs[i], sas[i], wqs[i], sws[i], y=ys[i], workspace=wss[i])

    step()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys:
            y.fill_(-1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(ys[i], eager[i]), (rep, i)
    # the replayed result is the oracle's, within the bf16 tolerance
    for i, (N, K) in enumerate(shapes):
        rwq, rsw = oq.quant_weight_blk128(bits16(ws[i]))
        rxq, rsa = oq.quant_act_tok128(bits16(xs[i]))
        ref64 = og.gemm_blockscaled(rxq, rsa, rwq, rsw, out="f64")
        ref = og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64))
        got = ys[i].float().cpu().numpy().astype(np.float64)
        assert_gemm_close(got, ref, ref64, "bf16", f"graph linear {i}")


def test_graph_replays_grouped_and_fused_calls():
    """The persistent grouped GEMM, its gathered bf16 form and the one-kernel GEMM on bf16
    activations (M <= 4), captured together (as the benchmark captures them): every replay equals
    the eager result."""
    counts, ids = synth.moe_routing(256, 8, 2, seed=620)
    off = synth.offsets_from_counts(counts).cuda()
    ids = ids.cuda()
    M = int(counts.sum())
    xt = synth.act_bf16(256, 1024, seed=621).cuda()
    x_rows = xt[ids.long()].contiguous()
    wq, sw = fq.quant_weight(synth.weight_bf16(8 * 512, 1024, seed=622).cuda())
    wq, sw = wq.view(8, 512, 1024), sw.view(8, 4, 8)
    xq, sa = fq.quant_act(x_rows)
    x_small = synth.act_bf16(3, 4096, seed=623).cuda()
    wd, swd = fq.quant_weight(synth.weight_bf16(4096, 4096, seed=624).cuda())
    y_g = torch.empty((M, 512), dtype=torch.bfloat16, device="cuda")
    y_f = torch.empty((M, 512), dtype=torch.bfloat16, device="cuda")
    y_s = torch.empty((3, 4096), dtype=torch.bfloat16, device="cuda")
    ws = fq.new_workspace(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GROUPED_GEMM_FUSED_ACT, M, 512,
                                                   1024, 8), "cuda")

    def step():
        fq.grouped_gemm(xq, sa, wq, sw, off, y=y_g)
        fq.grouped_gemm_fused_act(xt, wq, sw, off, row_ids=ids, y=y_f, workspace=ws)
        fq.gemm_fused_act(x_small, wd, swd, y=y_s)

    step()
    torch.cuda.synchronize()
    eager = [y.clone() for y in (y_g, y_f, y_s)]
    assert torch.equal(eager[0], eager[1])  # the gathered form gives the same bits
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for y in (y_g, y_f, y_s):
            y.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate((y_g, y_f, y_s)):
            assert torch.equal(y, eager[i]), (rep, i)
