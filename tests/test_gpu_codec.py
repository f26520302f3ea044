"""GPU parity of the device E4M3 encoder (fp8rl_encode_e4m3_f32) against the oracle's encoder.

Exhaustive over every non-negative float32 up to 464 (1,139,277,825 values) and, through the
sign symmetry the oracle is pinned to, over their negatives; plus the special values.
"""

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import fp8_blockwise_quantization_amd as fq
from oracle import e4m3
from tests import _codec_sweep

pytestmark = pytest.mark.gpu


def _gpu_codes(start: int, count: int, negate: bool) -> np.ndarray:
    bits = torch.arange(start, start + count, dtype=torch.int64, device="cuda").to(torch.int32)
    v = bits.view(torch.float32)
    if negate:
        v = -v
    return fq.encode_e4m3(v).cpu().numpy()


def test_encode_exhaustive_vs_oracle():
    work = list(_codec_sweep.chunks())
    workers = min(16, os.cpu_count() or 1)
    bad_pos = bad_neg = 0
    with ProcessPoolExecutor(max_workers=workers,
                             mp_context=multiprocessing.get_context("spawn")) as ex:
        for (start, count), ref in zip(work, ex.map(_codec_sweep.oracle_codes, *zip(*work))):
            bad_pos += int(np.count_nonzero(_gpu_codes(start, count, False) != ref))
            bad_neg += int(np.count_nonzero(_gpu_codes(start, count, True) != (ref | 0x80)))
    print(f"encoder sweep: {len(work)} chunks, mismatches +{bad_pos} -{bad_neg}", flush=True)
    assert bad_pos == 0 and bad_neg == 0


def test_encode_specials_and_tail():
    vals = np.array([0.0, -0.0, 448.0, -448.0, 448.00003, 463.99997, 464.0, 464.00003, 480.0,
                     1e30, -1e30, np.inf, -np.inf, np.nan, -np.nan, 2.0 ** -10, -(2.0 ** -10),
                     1.5 * 2.0 ** -9, 2.0 ** -149, -(2.0 ** -149), 3.0e-39], dtype=np.float32)
    got = fq.encode_e4m3(torch.from_numpy(vals).cuda()).cpu().numpy()
    want = e4m3.encode(vals)
    assert np.array_equal(got, want), (got, want)
    # lengths that are not a multiple of 4 take the scalar tail path
    for n in (1, 2, 3, 5, 7, 1021):
        v = torch.randn(n, generator=torch.Generator().manual_seed(n)) * 100
        got = fq.encode_e4m3(v.cuda()).cpu().numpy()
        assert np.array_equal(got, e4m3.encode(v.numpy()))
