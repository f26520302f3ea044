"""CPU oracle for the FP8 blockwise-quantized W8A8 linear layer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct CPU restatement of what
the GPU library computes. Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path (the HIP library and its Python binding) never does,
and the two share no code.

Sources (the pages this follows, cited by title and section):

* "Unified FP8: Moving Beyond Mixed Precision for Stable and Accelerated MoE RL" (LMSYS blog,
  digest), quick-read section: the two quantization equations S = max|X| / V_max and
  Q(x) = round(x / S), V_max being the largest FP8 value; the "FP8 scale choice" section: FP32
  scale factors (not E8M0).
* "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement Learning" (write-up),
  section 1 "dynamic weight sync": weights re-quantized every step in 128x128 blocks with one
  scale each, E4M3 with 4 exponent bits, 3 mantissa bits and range [-448, 448]; activations
  quantized dynamically.
* NVIDIA NeMo RL FP8 blog, "FP8 for linear layers in RL", Table 1: weights E4M3 with [128, 128]
  blocks, input activations E4M3 with [1, 128] groups, FP32 block scales.

Modules: ``e4m3`` (codec), ``quant`` (the two quantizers), ``gemm`` (dequantized fp64 GEMM and its
grouped-expert form), ``backward`` (the FP8 input- and weight-gradient GEMMs and the quantizations
they need) and ``kvcache`` (per-tensor Q/K/V scale recalibration and the FP8 KV-cache store).
Every function with no independent pin would say "parity unpinned"; none does at present (see the
tests under ``tests/test_oracle_*.py``).
"""

from . import backward, e4m3, gemm, kvcache, quant  # noqa: F401
