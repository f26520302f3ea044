"""Helpers shared by the GPU parity tests (host-side conversions and the GEMM tolerance)."""

from __future__ import annotations

import os

import numpy as np
import torch

#: Every tolerance check of this session: the worst |gpu - ref| / bound (the slack; <= 1 passes)
#: with the check's label and the test it ran in. conftest.py prints them at the end of the run.
SLACK: list = []


def _record(kind: str, what: str, out: str, shape, worst: float) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    SLACK.append({"test": test, "check": what, "kind": kind, "out": out,
                  "shape": [int(d) for d in shape], "slack": worst})


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def gemm_out_to_f64(y: torch.Tensor) -> np.ndarray:
    if y.dtype == torch.bfloat16:
        return y.float().cpu().numpy().astype(np.float64)
    return y.cpu().numpy().astype(np.float64)


def assert_gemm_close(got: np.ndarray, ref_rounded: np.ndarray, ref_f64: np.ndarray, out: str,
                      what: str = "") -> float:
    """Elementwise GEMM tolerance against the oracle.

    bf16 output: |gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref); float32 output: <= 1e-5 rms(ref);
    rms over the whole output matrix of the oracle's float64 result. Returns the worst ratio of
    error to bound (<= 1 passes).
    """
    rms = float(np.sqrt(np.mean(ref_f64 ** 2))) if ref_f64.size else 0.0
    err = np.abs(got - ref_rounded)
    if out == "bf16":
        bound = 2.0 ** -7 * np.abs(ref_rounded) + 1e-3 * rms
    else:
        bound = np.full(ref_rounded.shape, 1e-5 * rms)
    bound = np.maximum(bound, np.finfo(np.float64).tiny)
    ratio = err / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    _record("tolerance", what, out, got.shape, worst)
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(
            f"{what}: GEMM outside tolerance at {idx}: gpu={got[idx]!r} ref={ref_rounded[idx]!r} "
            f"err={err[idx]:.3e} bound={bound[idx]:.3e} (rms {rms:.3e}); "
            f"{int((ratio > 1).sum())} elements fail")
    return worst


def fp8_slice_bound(xq: np.ndarray, sa: np.ndarray, wq: np.ndarray, sw: np.ndarray,
                    b_rows: bool = False) -> np.ndarray:
    """Error bound of FP8-matrix-core slice sums (accum='fp8'), per output element.

    Model (measured on gfx950): the instruction aligns the 128 products of a slice to the largest
    one and truncates each below 2^(E - 14), E = floor(log2 max|p|), then combines its partial
    sums the same way. The slice error is then < 128 * 2^(E - 14) + 8 * 2^(E - 14) < 2^-6 max|p|,
    and max|p| <= max|dec(Xq[m, slice])| * max|dec(Wq[n, slice])|. Summed over slices with their
    scales: bound[m, n] = 2^-6 * sum_kb |sa[m,kb] sw[n/128,kb]| ax[m,kb] aw[n,kb].
    """
    from oracle import e4m3

    dec = np.abs(np.nan_to_num(e4m3.decode(np.arange(256)), nan=0.0))
    M, K = xq.shape
    N = wq.shape[0]
    KB = K // 128
    ax = dec[xq].reshape(M, KB, 128).max(axis=2) * np.abs(sa.astype(np.float64))
    # b_rows: sw holds one scale per row of B and slice ([N][KB]) instead of per 128x128 block
    swr = np.abs(sw.astype(np.float64)) if b_rows else np.repeat(np.abs(sw.astype(np.float64)), 128, axis=0)[:N]
    aw = dec[wq].reshape(N, KB, 128).max(axis=2) * swr
    return 2.0 ** -6 * (ax @ aw.T)


def assert_within(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str) -> float:
    err = np.abs(got - ref)
    ratio = err / np.maximum(bound, np.finfo(np.float64).tiny)
    worst = float(ratio.max()) if ratio.size else 0.0
    _record("bound", what, "", got.shape, worst)
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: outside bound at {idx}: gpu={got[idx]!r} ref={ref[idx]!r} "
                             f"bound={bound[idx]:.3e}")
    return worst
