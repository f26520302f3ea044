"""The no-allocation GEMM entry point (fp8rl_gemm_w8a8_blockscaled_noalloc) against the workspace
entry point (fp8rl_gemm_w8a8_blockscaled), both called through the C ABI with raw device pointers,
and against the oracle.

Four calls in a row share the library's static scratch: mid-M shapes whose K is split over
workgroups (partials in the scratch, summed by a second kernel), the later ones smaller than the
first, then a decode shape (K split over workgroups too: arrival counters and partials in the
scratch); each result must equal the workspace form's bit for bit and meet the GEMM tolerance
against the oracle.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import assert_gemm_close, bits16, gemm_out_to_f64, to_dev_f32, to_dev_u8
from workloads import synth

pytestmark = pytest.mark.gpu

SHAPES = [(300, 768, 2048), (200, 1024, 4096), (130, 512, 1024), (64, 4096, 4096)]


def _operands(M, N, K, seed):
    x = synth.act_bf16(M, K, seed=seed)
    w = synth.weight_bf16(N, K, seed=seed + 1, outlier_frac=0.001)
    xq, sa = oq.quant_act_tok128(bits16(x))
    wq, sw = oq.quant_weight_blk128(bits16(w))
    return xq, sa, wq, sw


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_noalloc_equals_workspace_entry_point(out):
    L = fq.lib()
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    code = 0 if out == "bf16" else 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i, (M, N, K) in enumerate(SHAPES):
        print(f"[noalloc] call {i}: {M}x{N}x{K} out={out}", flush=True)
        assert fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, M, N, K) > 0  # uses the scratch
        xq, sa, wq, sw = _operands(M, N, K, 7700 + 10 * i)
        d = [to_dev_u8(xq), to_dev_f32(sa), to_dev_u8(wq), to_dev_f32(sw)]
        ptrs = [ctypes.c_void_p(t.data_ptr()) for t in d]
        y_ref = torch.full((M, N), 5.0, dtype=dt, device="cuda")
        need = L.fp8rl_workspace_bytes(0, M, N, K, 0)
        ws = fq.new_workspace(need, "cuda")  # (a zeroed header even when need is 0)
        st = L.fp8rl_gemm_w8a8_blockscaled(*ptrs, M, N, K, ctypes.c_void_p(y_ref.data_ptr()), code,
                                           N, 3, ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream)
        assert st == 0
        y = torch.full((M, N + 8), 9.0, dtype=dt, device="cuda")  # pitch N + 8, canary columns
        st = L.fp8rl_gemm_w8a8_blockscaled_noalloc(*ptrs, M, N, K, ctypes.c_void_p(y.data_ptr()),
                                                   code, N + 8, 3, stream)
        assert st == 0
        torch.cuda.synchronize()
        assert torch.equal(y[:, :N], y_ref), f"call {i}: no-alloc and workspace results differ"
        assert torch.all(y[:, N:] == 9.0)
        ref64 = og.gemm_blockscaled(xq, sa, wq, sw, out="f64")
        ref = (og.bf16_bits_to_f64(og.round_f64_to_bf16_bits(ref64)) if out == "bf16"
               else ref64.astype(np.float32).astype(np.float64))
        assert_gemm_close(gemm_out_to_f64(y[:, :N].contiguous()), ref, ref64, out,
                          f"noalloc {M}x{N}x{K}")


def test_noalloc_binding_and_scratch_limit():
    xq, sa, wq, sw = _operands(64, 1024, 4096, 7790)
    d = [to_dev_u8(xq), to_dev_f32(sa), to_dev_u8(wq), to_dev_f32(sw)]
    y = torch.empty((64, 1024), dtype=torch.bfloat16, device="cuda")
    fq.gemm_noalloc(*d, y=y)
    ref = fq.gemm(*d)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    # a shape whose split partials exceed the static scratch is refused with FP8RL_ERR_SCRATCH
    M, N, K = 1024, 1152, 65536
    big = [torch.zeros((M, K), dtype=torch.uint8, device="cuda"),
           torch.ones((M, K // 128), dtype=torch.float32, device="cuda"),
           torch.zeros((N, K), dtype=torch.uint8, device="cuda"),
           torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")]
    yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fq.Fp8rlError) as e:
        fq.gemm_noalloc(*big, y=yb)
    assert e.value.status == 8
