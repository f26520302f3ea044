"""GPU parity of the 128x128 weight and 1x128 activation quantizers against the oracle.

Codes and scales must be bit-exact. Inputs are the seeded synthetic tensors of the workloads
(weights N(0, 0.02) with 0.1 % x10 outliers, activations N(0, 1) with 1 % x20 outlier channels),
full-size for the Qwen3-8B decoder block and its prefill activations, plus hand-built edge blocks.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import quant as oq
from tests.gpu_util import bits16
from workloads import synth

pytestmark = pytest.mark.gpu


def _check_weight(w: torch.Tensor, what: str):
    print(f"[quant_weight] {what} {tuple(w.shape)}", flush=True)
    wq, sw = fq.quant_weight(w.cuda())
    torch.cuda.synchronize()
    rq, rs = oq.quant_weight_blk128(bits16(w))
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), rs.view(np.uint32)), f"{what}: scales"
    got = wq.cpu().numpy()
    bad = int(np.count_nonzero(got != rq))
    assert bad == 0, f"{what}: {bad} codes differ"


def _check_act(x: torch.Tensor, what: str):
    print(f"[quant_act] {what} {tuple(x.shape)}", flush=True)
    xq, sa = fq.quant_act(x.cuda())
    torch.cuda.synchronize()
    rq, rs = oq.quant_act_tok128(bits16(x))
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), rs.view(np.uint32)), f"{what}: scales"
    bad = int(np.count_nonzero(xq.cpu().numpy() != rq))
    assert bad == 0, f"{what}: {bad} codes differ"


def test_tiny_config():
    _check_weight(synth.weight_bf16(256, 256, seed=synth.seed_of(1, 0)), "tiny W")
    _check_act(synth.act_bf16(4, 256, seed=synth.seed_of(1, 1)), "tiny X")


@pytest.mark.parametrize("idx", range(7))
def test_qwen3_8b_block_weights_full(idx):
    name, N, K = synth.DENSE_LINEARS_QWEN3_8B[idx]
    w = synth.weight_bf16(N, K, seed=synth.seed_of(2, idx), outlier_frac=0.001)
    _check_weight(w, name)


@pytest.mark.parametrize("M,K", [(64, 4096), (64, 12288), (8192, 4096), (8192, 12288), (67, 384),
                                 (1, 128), (257, 1024)])
def test_activations(M, K):
    _check_act(synth.act_bf16(M, K, seed=synth.seed_of(3, M, K)), f"X[{M}][{K}]")


def _edge_weight() -> torch.Tensor:
    """A 384x512 weight whose 3x4 blocks each exercise one edge case."""
    g = torch.Generator().manual_seed(77)
    w = (torch.randn((384, 512), generator=g) * 0.02).to(torch.bfloat16)
    b = lambda i, j: w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
    b(0, 0).zero_()                                   # all-zero block: S = 1, all codes 0
    b(0, 1).zero_()
    b(0, 1)[5, 7] = -3.25                             # one nonzero element -> 0xFE
    b(0, 2).fill_(0.015625)                           # constant block -> all 0x7E
    b(0, 3).copy_(-b(0, 3).abs())                     # all negative
    b(1, 0).mul_(2.0 ** -130)                         # bf16 subnormals: subnormal float32 S
    b(1, 1).zero_()
    b(1, 1)[0, 0] = -0.0                              # negative zero keeps its sign
    b(1, 2).mul_(1e30)                                # huge magnitudes
    b(1, 3).copy_(torch.full_like(b(1, 3), 3.389e38))  # near the bf16 maximum
    b(2, 0)[:, :] = torch.tensor(0.0703125).to(torch.bfloat16)  # constant, exact grid value
    b(2, 0)[3, 3] = 3.5                               # amax 3.5 -> S = 2^-7 exactly; ties at x*128
    b(2, 0)[4, :19] = torch.tensor([3.5, 1.0, -2.0, 0.25, 0.30078125, 0.0703125, 0.06640625,
                                    0.07421875, 2.0 ** -16, 2.0 ** -17, -(2.0 ** -17),
                                    3 * 2.0 ** -17, -0.0, 0.0, -3.5, 2.0 ** -13, 15 * 2.0 ** -17,
                                    3.375, 3.25]).to(torch.bfloat16)
    b(2, 1).mul_(2.0 ** -100)                         # tiny but normal
    return w


def test_edge_blocks():
    _check_weight(_edge_weight(), "edge blocks")
    _check_act(_edge_weight(), "edge blocks as activation rows")


def test_strided_rows_and_canaries():
    """Row pitches larger than K: padding bytes of the outputs must be left untouched."""
    N, K, pad = 256, 384, 64
    w_full = synth.weight_bf16(N, K + pad, seed=91)
    w = w_full[:, :K].cuda()  # pitch K + pad
    wq_full = torch.full((N, K + 32), 0xA5, dtype=torch.uint8, device="cuda")
    # K / 128 = 3 is odd: the last 128x256 strip of each block row holds one block; the scales
    # are followed by canaries that no missing right block may touch
    nsw = (N // 128) * (K // 128)
    sw_full = torch.full((nsw + 8,), -7.0, dtype=torch.float32, device="cuda")
    sw = sw_full[:nsw].view(N // 128, K // 128)
    fq.quant_weight(w, wq_full[:, :K], sw)
    torch.cuda.synchronize()
    assert torch.all(wq_full[:, K:] == 0xA5)
    assert torch.all(sw_full[nsw:] == -7.0)
    rq, rs = oq.quant_weight_blk128(bits16(w_full[:, :K]))
    assert np.array_equal(wq_full[:, :K].cpu().numpy(), rq)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    x_full = synth.act_bf16(37, K + pad, seed=92)
    x = x_full[:, :K].cuda()
    xq_full = torch.full((37, K + 16), 0x5A, dtype=torch.uint8, device="cuda")
    sa = torch.empty((37, K // 128), dtype=torch.float32, device="cuda")
    fq.quant_act(x, xq_full[:, :K], sa)
    torch.cuda.synchronize()
    assert torch.all(xq_full[:, K:] == 0x5A)
    rq, rs = oq.quant_act_tok128(bits16(x_full[:, :K]))
    assert np.array_equal(xq_full[:, :K].cpu().numpy(), rq)
    assert np.array_equal(sa.cpu().numpy(), rs)


def test_zero_rows_is_a_noop_and_deterministic():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    xq, sa = fq.quant_act(x)
    assert xq.shape == (0, 256)
    w = synth.weight_bf16(1024, 2048, seed=93).cuda()
    a1, s1 = fq.quant_weight(w)
    a2, s2 = fq.quant_weight(w)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(s1, s2)


def test_batched_weights_one_launch_per_32():
    """40 matrices (more than one launch) plus empty ones through the batched entry point."""
    shapes = [(128 * (1 + i % 3), 128 * (1 + (i * 7) % 4)) for i in range(40)]
    ws = [synth.weight_bf16(N, K, seed=500 + i, outlier_frac=0.001).cuda()
          for i, (N, K) in enumerate(shapes)]
    wqs = [torch.empty((N, K), dtype=torch.uint8, device="cuda") for N, K in shapes]
    sws = [torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda") for N, K in shapes]
    empty_w = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    empty_q = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    empty_s = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    fq.quant_weights(ws[:20] + [empty_w] + ws[20:], wqs[:20] + [empty_q] + wqs[20:],
                     sws[:20] + [empty_s] + sws[20:])
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        rq, rs = oq.quant_weight_blk128(bits16(w))
        assert np.array_equal(wqs[i].cpu().numpy(), rq), i
        assert np.array_equal(sws[i].cpu().numpy().view(np.uint32), rs.view(np.uint32)), i


def test_batched_qwen3_block_matches_single_calls():
    ws = [synth.weight_bf16(N, K, seed=synth.seed_of(2, i), outlier_frac=0.001).cuda()
          for i, (_, N, K) in enumerate(synth.DENSE_LINEARS_QWEN3_8B)]
    wqs = [torch.empty(w.shape, dtype=torch.uint8, device="cuda") for w in ws]
    sws = [torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.float32, device="cuda")
           for w in ws]
    fq.quant_weights(ws, wqs, sws)
    for i, w in enumerate(ws):
        a, b = fq.quant_weight(w)
        torch.cuda.synchronize()
        assert torch.equal(a, wqs[i]) and torch.equal(b, sws[i])
    # and against the oracle for the smallest one
    rq, rs = oq.quant_weight_blk128(bits16(ws[1]))
    assert np.array_equal(wqs[1].cpu().numpy(), rq)
