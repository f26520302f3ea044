"""Helpers shared by the GPU parity tests (host-side conversions and the GEMM tolerance)."""

from __future__ import annotations

import numpy as np
import torch


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
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(
            f"{what}: GEMM outside tolerance at {idx}: gpu={got[idx]!r} ref={ref_rounded[idx]!r} "
            f"err={err[idx]:.3e} bound={bound[idx]:.3e} (rms {rms:.3e}); "
            f"{int((ratio > 1).sum())} elements fail")
    return worst
