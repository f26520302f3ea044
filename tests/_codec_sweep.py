"""Chunked sweeps over float32 bit patterns for the exhaustive encoder checks (test helper)."""

from __future__ import annotations

import numpy as np

# Non-negative float32 bit patterns 0 .. 0x43E80000 (= 464.0) inclusive: the range where torch's
# float8_e4m3fn cast (round to nearest even, NaN above 464) and a saturating encoder must agree.
LAST_NONNEG_BITS = 0x43E80000
CHUNK = 1 << 23


def chunks(last=LAST_NONNEG_BITS, chunk=CHUNK):
    start = 0
    while start <= last:
        n = min(chunk, last - start + 1)
        yield start, n
        start += n


def oracle_codes(start: int, count: int) -> np.ndarray:
    from oracle import e4m3

    bits = np.arange(start, start + count, dtype=np.uint64).astype(np.uint32)
    return e4m3.encode(bits.view(np.float32))


def torch_codes(start: int, count: int) -> np.ndarray:
    import torch

    bits = np.arange(start, start + count, dtype=np.uint64).astype(np.uint32)
    v = torch.from_numpy(bits.view(np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def mismatches_vs_torch(args) -> int:
    import torch

    torch.set_num_threads(1)
    start, count = args
    return int(np.count_nonzero(oracle_codes(start, count) != torch_codes(start, count)))
