"""Pins for the oracle's per-tensor (KV cache / Q/K/V) quantizer (CPU only).

Independent references: a tensor worked by hand (golden fixture), torch's own float8_e4m3fn cast
for in-range quotients, the exact rational quotient for the scale, brute-force maxima on tiny
tensors, the reduction to the (separately pinned) 1x128 group quantizer when the tensor is a
single group, and closed forms for saturation.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, kvcache, quant
from tests.exact import f32_to_fraction
from tests.test_oracle_quant import bf16_bits, random_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_tensor():
    d = json.load(open(os.path.join(GOLDEN, "worked_kv_tensor.json")))
    a = np.float32(0.0)
    for batch in d["calibration_batches"]:
        a = kvcache.amax_accumulate(a, bf16_bits([float(v) for v in batch]))
    assert a == np.float32(d["amax"])
    S = kvcache.scale_per_tensor(a)
    assert S == np.float32(d["scale"])
    xs = [float(e["x"]) for e in d["entries"]]
    q = kvcache.quant_per_tensor(bf16_bits(xs).reshape(1, -1), S)
    want = [int(e["code"], 16) for e in d["entries"]]
    assert q.ravel().tolist() == want
    for e in d["entries"]:  # the fixture's quotients are the exact x / S
        assert Fraction(e["x"]) / Fraction(d["scale"]) == Fraction(e["x_over_S"].replace("-0", "0"))


def test_amax_brute_force_and_running_max():
    batches = [random_bf16((3, 5), seed=s, scale=10.0 ** (s - 2)) for s in range(4)]
    running = np.float32(0.0)
    best = 0.0
    for b in batches:
        running = kvcache.amax_accumulate(running, b)
        for v in quant.bf16_bits_to_f32(b).ravel().tolist():  # element by element
            best = max(best, abs(v))
        assert running == np.float32(best)
    assert kvcache.amax(np.zeros((0, 4), np.uint16)) == 0


@pytest.mark.parametrize("amax", [3.5, 1.0, 0.0, 2.0 ** -133, 3.3895313892515355e38, 0.1])
def test_scale_is_the_correctly_rounded_quotient(amax):
    S = kvcache.scale_per_tensor(np.float32(amax))
    if amax == 0.0:
        assert S == 1
        return
    exact = f32_to_fraction(np.float32(amax)) / 448
    # S is a float32 nearest to amax / 448: no float32 lies strictly closer
    s = f32_to_fraction(S)
    for nb in (np.nextafter(S, np.float32(0)), np.nextafter(S, np.float32(np.inf))):
        assert abs(f32_to_fraction(nb) - exact) >= abs(s - exact)


def test_matches_torch_cast_in_range():
    # quotients within +-448 (calibrated on the tensor itself): torch's float8_e4m3fn cast of the
    # float32 quotient is an independent encoder
    for seed in range(6):
        x = random_bf16((33, 160), seed=100 + seed, scale=10.0 ** (seed - 3))
        S = kvcache.scale_per_tensor(kvcache.amax(x))
        q = kvcache.quant_per_tensor(x, S)
        t = torch.from_numpy(quant.bf16_bits_to_f32(x)) / torch.tensor(S, dtype=torch.float32)
        ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, ref)


def test_single_group_tensor_equals_group_quantizer():
    for seed in range(5):
        x = random_bf16((1, 128), seed=200 + seed, scale=3.0)
        S = kvcache.scale_per_tensor(kvcache.amax(x))
        q = kvcache.quant_per_tensor(x, S)
        qg, sg = quant.quant_act_tok128(x)
        assert sg[0, 0] == S and np.array_equal(q, qg)


def test_saturation_beyond_calibrated_range():
    S = np.float32(2.0 ** -7)  # calibrated amax 3.5
    x = bf16_bits([3.75, -8.0, 2.0 ** 100, -(2.0 ** 127), 3.5, -3.625])
    q = kvcache.quant_per_tensor(x.reshape(1, -1), S).ravel()
    # 480, -1024, 2^107, overflow to -inf all saturate; 448 exact; -464 saturates to -448
    assert q.tolist() == [0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0xFE]
    tiny = np.float32(2.0 ** -140)  # a float32 subnormal scale: 1.0 / S overflows float32
    assert kvcache.quant_per_tensor(bf16_bits([1.0, -1.0]).reshape(1, -1), tiny).ravel().tolist() == [0x7E, 0xFE]


def test_codes_dequantize_within_half_step():
    x = random_bf16((64, 256), seed=7, scale=0.5)
    S = kvcache.scale_per_tensor(kvcache.amax(x))
    q = kvcache.quant_per_tensor(x, S)
    v = quant.bf16_bits_to_f32(x).astype(np.float64) / float(S)
    d = e4m3.decode(q)
    # nearest-even on the E4M3 grid: error at most half the local spacing (2^(e-3) / 2, >= 2^-10)
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    assert np.all(np.abs(d - v) <= 2.0 ** (e - 4) + 1e-300)


def test_kv_cache_store_slots():
    cache = np.full((10, 16), 0xAA, dtype=np.uint8)
    x = random_bf16((4, 16), seed=3)
    S = kvcache.scale_per_tensor(kvcache.amax(x))
    q = kvcache.quant_per_tensor(x, S)
    out = kvcache.kv_cache_store(cache, x, S, slot=[7, -1, 0, 3])
    assert np.array_equal(out[7], q[0]) and np.array_equal(out[0], q[2]) and np.array_equal(out[3], q[3])
    untouched = [r for r in range(10) if r not in (7, 0, 3)]
    assert np.all(out[untouched] == 0xAA)
    assert np.all(cache == 0xAA)  # the input cache is not modified
    out2 = kvcache.kv_cache_store(cache, x, S)
    assert np.array_equal(out2[:4], q) and np.all(out2[4:] == 0xAA)
    narrow = kvcache.kv_cache_store(cache, x[:, :8], S, slot=[1, 2, 3, 4])
    assert np.array_equal(narrow[1:5, :8], kvcache.quant_per_tensor(x[:, :8], S))
    assert np.all(narrow[1:5, 8:] == 0xAA)


def test_rejects_bad_scale_and_nonfinite():
    x = bf16_bits([1.0, 2.0]).reshape(1, -1)
    for S in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            kvcache.quant_per_tensor(x, np.float32(S))
    bad = np.array([[0x7F80]], dtype=np.uint16)  # +inf
    with pytest.raises(ValueError):
        kvcache.amax(bad)
