"""GPU parity of the per-tensor FP8 path (Q/K/V activations and the KV cache) against the oracle.

Everything is integer or exactly rounded here, so every result must be bit-exact: the running
amax, the scale (an IEEE float32 division), and every code, including rows skipped or redirected
by the slot mapping and the bytes around them. Inputs are seeded synthetic K/V-shaped activations
(Qwen3-8B: 8 KV heads x 128 = 1024 columns, 32 query heads = 4096 columns, fused Q/K/V rows of
6144), N(0, 1) with 1 % x20 outlier channels.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import kvcache as ok
from tests.gpu_util import bits16
from workloads import synth

pytestmark = pytest.mark.gpu


def _f32_bits(t) -> np.ndarray:
    return np.asarray(t, dtype=np.float32).view(np.uint32)


def _check_amax(x: torch.Tensor, what: str):
    print(f"[amax] {what} {tuple(x.shape)} ld={x.stride(0)}", flush=True)
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    fq.amax(x, a)
    torch.cuda.synchronize()
    want = ok.amax(bits16(x))
    assert _f32_bits(a.cpu().numpy()[0]) == _f32_bits(want), what


@pytest.mark.parametrize("T,C", [(1, 8), (3, 24), (64, 1024), (4097, 1024), (16384, 1024),
                                 (8192, 4096)])
def test_amax_dense(T, C):
    _check_amax(synth.act_bf16(T, C, seed=synth.seed_of(20, T, C)).cuda(), f"x[{T}][{C}]")


def test_amax_column_slices_of_fused_qkv():
    qkv = synth.act_bf16(3000, 6144, seed=synth.seed_of(21, 0)).cuda()
    for name, lo, hi in (("q", 0, 4096), ("k", 4096, 5120), ("v", 5120, 6144)):
        _check_amax(qkv[:, lo:hi], f"{name} slice")


def test_amax_accumulates_across_batches_and_ignores_sign():
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    want = np.float32(0.0)
    for b in range(4):
        x = synth.act_bf16(700 + 13 * b, 1024, seed=synth.seed_of(22, b)) * (0.5 + b)
        if b == 2:
            x[5, 7] = -1000.0  # a negative extreme decides the amax
        fq.amax(x.cuda(), a)
        want = ok.amax_accumulate(want, bits16(x))
    torch.cuda.synchronize()
    assert _f32_bits(a.cpu().numpy()[0]) == _f32_bits(want)
    assert float(want) == 1000.0


def test_amax_batched_many_tensors():
    # Q, K, V of 36 layers: 108 tensors, more than one launch's worth
    T = 256
    xs, want = [], []
    for layer in range(36):
        qkv = synth.act_bf16(T, 6144, seed=synth.seed_of(23, layer)).cuda() * (1 + layer % 5)
        for lo, hi in ((0, 4096), (4096, 5120), (5120, 6144)):
            xs.append(qkv[:, lo:hi])
            want.append(ok.amax(bits16(qkv[:, lo:hi])))
    amax = torch.zeros(len(xs), dtype=torch.float32, device="cuda")
    print(f"[amax batched] {len(xs)} tensors", flush=True)
    fq.amax_batched(xs, amax)
    torch.cuda.synchronize()
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), np.array(want, np.float32).view(np.uint32))


def test_scale_from_amax_is_ieee_division():
    vals = [0.0, 3.5, 1.0, 0.1, 1000.0, 3.3895313892515355e38, 2.0 ** -133, 7 * 2.0 ** -144,
            5 * 2.0 ** -140, 1e-40, 448.0, 12345.678]
    rng = np.random.default_rng(5)
    vals += list(np.abs(rng.standard_normal(2000)).astype(np.float32) *
                 np.float32(2.0) ** rng.integers(-149, 100, 2000).astype(np.float32))
    a = np.array(vals, dtype=np.float32)
    a = a[np.isfinite(a)]
    s = fq.scale_from_amax(torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    want = np.array([ok.scale_per_tensor(v) for v in a], dtype=np.float32)
    got = s.cpu().numpy()
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, [(float(a[i]), float(got[i]), float(want[i])) for i in bad[:5]]


def _check_quant(x: torch.Tensor, S: np.float32, what: str, out_rows=None, slot=None, ld_out=None):
    T, C = x.shape
    out_rows = T if out_rows is None else out_rows
    ld_out = C if ld_out is None else ld_out
    print(f"[quant per tensor] {what} {tuple(x.shape)} -> [{out_rows}][{ld_out}]", flush=True)
    canary = np.random.default_rng(1).integers(0, 256, (out_rows, ld_out), dtype=np.uint8)
    out = torch.from_numpy(canary.copy()).cuda()
    sl = None if slot is None else torch.tensor(slot, dtype=torch.int64, device="cuda")
    fq.quant_per_tensor(x, torch.tensor([S], dtype=torch.float32, device="cuda"), out, sl)
    torch.cuda.synchronize()
    # the oracle's store skips slots past the cache like the kernel does (rows >= out_rows)
    slots = None if slot is None else [s if s < out_rows else -1 for s in slot]
    want = ok.kv_cache_store(canary, bits16(x), S, slot=slots)
    got = out.cpu().numpy()
    bad = int(np.count_nonzero(got != want))
    assert bad == 0, f"{what}: {bad} bytes differ"


@pytest.mark.parametrize("T,C", [(1, 8), (5, 136), (64, 1024), (12288, 1024), (16384, 1024),
                                 (32768, 1024), (8192, 4096)])
def test_quant_self_calibrated(T, C):
    x = synth.act_bf16(T, C, seed=synth.seed_of(24, T, C)).cuda()
    S = ok.scale_per_tensor(ok.amax(bits16(x)))
    _check_quant(x, S, "self-calibrated")


def test_quant_saturates_beyond_calibration_and_tiny_scales():
    x = synth.act_bf16(512, 1024, seed=synth.seed_of(25, 0)).cuda()
    calib = synth.act_bf16(512, 1024, seed=synth.seed_of(25, 1))
    S = ok.scale_per_tensor(ok.amax(bits16(calib)) / np.float32(4.0))  # a quarter of the range
    _check_quant(x, S, "scale from other data")
    y = x.clone()
    y[0, :8] = torch.tensor([1e30, -1e30, 3e38, -3e38, 0.0, -0.0, 1e-30, -1e-30]).to(torch.bfloat16)
    _check_quant(y, np.float32(2.0 ** -140), "subnormal scale")


def test_quant_into_cache_with_slots():
    T, C, rows = 300, 1024, 1000
    x = synth.act_bf16(T, C, seed=synth.seed_of(26, 0)).cuda()
    S = ok.scale_per_tensor(ok.amax(bits16(x)))
    perm = np.random.default_rng(3).permutation(rows)[:T].tolist()
    perm[7] = -1
    perm[11] = rows      # past the cache: skipped
    perm[12] = rows + 5  # past the cache: skipped
    perm[13] = -100
    _check_quant(x, S, "slots", out_rows=rows, slot=perm)
    _check_quant(x, S, "slots, wider cache rows", out_rows=rows, slot=perm, ld_out=1032)


def test_quant_column_slice_and_pitch():
    qkv = synth.act_bf16(777, 6144, seed=synth.seed_of(27, 0)).cuda()
    k = qkv[:, 4096:5120]
    S = ok.scale_per_tensor(ok.amax(bits16(k)))
    _check_quant(k, S, "k slice of fused qkv", ld_out=2048)


def test_recalibration_step_on_device():
    # amax over two calibration batches -> scales -> quantize new K/V rows into a cache, with no
    # host round trip between the calls
    T, C = 2048, 1024
    cal = [synth.act_bf16(T, 2 * C, seed=synth.seed_of(28, b)).cuda() for b in range(2)]
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    for c in cal:
        fq.amax_batched([c[:, :C], c[:, C:]], amax)
    scale = fq.scale_from_amax(amax)
    new = synth.act_bf16(64, 2 * C, seed=synth.seed_of(28, 9)).cuda() * 1.5
    slot = torch.arange(100, 164, dtype=torch.int64, device="cuda")
    kc = torch.zeros((256, C), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((256, C), dtype=torch.uint8, device="cuda")
    fq.quant_per_tensor(new[:, :C], scale[0:1], kc, slot)
    fq.quant_per_tensor(new[:, C:], scale[1:2], vc, slot)
    torch.cuda.synchronize()
    want_a = [np.float32(0.0), np.float32(0.0)]
    for c in cal:
        want_a[0] = ok.amax_accumulate(want_a[0], bits16(c[:, :C]))
        want_a[1] = ok.amax_accumulate(want_a[1], bits16(c[:, C:]))
    want_s = [ok.scale_per_tensor(a) for a in want_a]
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), np.array(want_s, np.float32).view(np.uint32))
    zero = np.zeros((256, C), np.uint8)
    s = list(range(100, 164))
    assert np.array_equal(kc.cpu().numpy(), ok.kv_cache_store(zero, bits16(new[:, :C]), want_s[0], s))
    assert np.array_equal(vc.cpu().numpy(), ok.kv_cache_store(zero, bits16(new[:, C:]), want_s[1], s))


def test_quant_batched_k_and_v_of_many_layers():
    # each layer's new K and V rows in one descriptor pair; 40 descriptors = 3 launches
    T, C, rows = 333, 1024, 600
    layers = 20
    rng = np.random.default_rng(8)
    xs, scales, outs, slots, want = [], [], [], [], []
    for l in range(layers):
        kv = synth.act_bf16(T, 2 * C, seed=synth.seed_of(29, l)).cuda() * (1 + l % 3)
        slot = rng.permutation(rows)[:T].astype(np.int64)
        slot[::17] = -1
        sl = torch.from_numpy(slot).cuda()
        for half in (kv[:, :C], kv[:, C:]):
            S = ok.scale_per_tensor(ok.amax(bits16(half)) * np.float32(0.75))
            canary = np.full((rows, C), 0x5A, np.uint8)
            xs.append(half)
            scales.append(torch.tensor([S], dtype=torch.float32, device="cuda"))
            outs.append(torch.from_numpy(canary.copy()).cuda())
            slots.append(sl)
            want.append(ok.kv_cache_store(canary, bits16(half), S, slot=slot.tolist()))
    print(f"[quant batched] {len(xs)} tensors", flush=True)
    fq.quant_per_tensor_batched(xs, scales, outs, slots)
    torch.cuda.synchronize()
    for i, (o, w) in enumerate(zip(outs, want)):
        assert np.array_equal(o.cpu().numpy(), w), f"descriptor {i}"
