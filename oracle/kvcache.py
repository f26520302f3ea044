"""Per-tensor FP8 for attention Q/K/V activations and the stored KV cache. TEST INFRASTRUCTURE.

What the pages fix:

* NeMo RL FP8 blog, section on extending FP8 to the KV cache and attention, and its Table 3: the
  Q/K/V attention activations and the stored KV cache are E4M3 with one FP32 scale per tensor;
  because the policy weights change every step, the trainer recomputes the Q/K/V scales at the
  end of each step from data run through the updated weights, and the new scales are handed to
  the inference engine for the next rollout;
* FP8-RL write-up, section 4 (KV-cache compression), and the arXiv listing's abstract: the same
  per-step recalibration of the QKV scales, either inside the engine or on the trainer side;
* the quantization rule itself (Unified FP8 blog, quick-read section): S = max|X| / V_max and
  Q(x) = round(x / S), with V_max = 448 for E4M3 (FP8-RL write-up, section 1).

Readings where the pages leave a step open (each also listed in the design notes):

* T1: the per-tensor scale uses the block quantizer's rule (Q2-Q4 of oracle.quant):
  S = fp32(amax / 448), S = 1 when amax == 0; amax is the largest |x| over every calibration
  batch of that tensor (the running maximum of the per-batch maxima);
* T2: the element step is also the block quantizer's: code = E4M3_RNE_sat(fp32(x) / S) with the
  IEEE float32 quotient;
* T3: a value larger than the calibrated amax (the scale was fitted on other data) saturates to
  +-448, as does a quotient that overflows float32;
* T4: storing new rows into the cache: row r of the new tokens goes to cache row slot[r]; a
  negative slot skips the row; without a slot array row r goes to cache row r.
"""

from __future__ import annotations

import numpy as np

from . import e4m3
from .quant import bf16_bits_to_f32, scale_from_amax


def _finite_f32(bits) -> np.ndarray:
    x32 = bf16_bits_to_f32(bits)
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    return x32


def amax(bits) -> np.float32:
    """Largest |x| over all elements of a bf16 tensor (exact); 0 for an empty tensor."""
    x32 = _finite_f32(bits)
    return np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)


def amax_accumulate(prev, bits) -> np.float32:
    """T1: running amax over calibration batches: max(prev, amax(batch))."""
    return np.float32(max(np.float32(prev), amax(bits)))


def scale_per_tensor(a) -> np.float32:
    """T1: S = fp32(amax / 448), 1 when amax == 0."""
    return np.float32(scale_from_amax(np.float32(a)))


def quant_per_tensor(bits, S) -> np.ndarray:
    """T2/T3: E4M3 codes of fp32(x) / S for every element (S a positive finite float32)."""
    S = np.float32(S)
    if not (np.isfinite(S) and S > 0):
        raise ValueError("the per-tensor scale must be positive and finite")
    x32 = _finite_f32(bits)
    with np.errstate(over="ignore"):  # float32 overflow -> inf -> saturates to +-448
        q = (x32 / S).astype(np.float32)
    return e4m3.encode(q)


def kv_cache_store(cache, bits, S, slot=None) -> np.ndarray:
    """T4: a copy of `cache` (uint8 [rows][cols]) with the quantized new rows written at their
    slots; `bits` is bf16 [T][cols'] with cols' <= cols (the first cols' bytes of a row)."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    q = quant_per_tensor(bits, S)
    T = q.shape[0]
    rows = np.arange(T) if slot is None else np.asarray(slot, dtype=np.int64)
    if rows.shape != (T,):
        raise ValueError("one slot per new row")
    for r in range(T):
        if rows[r] >= 0:
            out[rows[r], :q.shape[1]] = q[r]
    return out
