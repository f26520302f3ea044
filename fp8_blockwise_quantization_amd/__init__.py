"""MI355X (gfx950) FP8 blockwise-quantized W8A8 linear layer.

Python face of ``libfp8rl.so``: 128x128 weight re-quantization, 1x128 per-token activation
quantization, the blockwise-scaled FP8 GEMM and its grouped-expert (MoE) form, and per-tensor
FP8 for attention Q/K/V and the KV cache with recalibrated scales, and the quantizers and GEMM
of the FP8 backward pass (transposed weight copy, 128x1 token groups, row-scaled GEMM), and the
GEMMs with the activation quantization fused in (dense, and grouped with the codes read through
the router's token indices). Tensors live on the GPU; the functions only marshal arguments into
the C ABI (include/fp8rl.h).
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    FP8RL_ACCUM_AUTO,
    FP8RL_ACCUM_F16,
    FP8RL_ACCUM_FP8,
    FP8RL_ACCUM_MX,
    FP8RL_OP_GEMM,
    FP8RL_OP_GEMM_FUSED_ACT,
    FP8RL_OP_GEMM_ROWSCALED,
    FP8RL_OP_GROUPED_GEMM,
    FP8RL_OP_GROUPED_GEMM_FUSED_ACT,
    FP8RL_OUT_BF16,
    FP8RL_OUT_F32,
    FP8RL_SCALE_FP32,
    FP8RL_SCALE_POW2,
    Fp8rlError,
    fp8rl_amax_bf16,
    fp8rl_amax_bf16_batched,
    fp8rl_encode_e4m3_f32,
    fp8rl_gemm_w8a8_blockscaled,
    fp8rl_gemm_w8a8_blockscaled_noalloc,
    fp8rl_gemm_w8a8_fused_act_quant,
    fp8rl_gemm_w8a8_rowscaled,
    fp8rl_grouped_gemm_w8a8,
    fp8rl_grouped_gemm_w8a8_fused_act_quant,
    fp8rl_quant_act_colwise128,
    fp8rl_quant_act_tok128,
    fp8rl_quant_bf16_per_tensor,
    fp8rl_quant_bf16_per_tensor_batched,
    fp8rl_quant_act_tok128_ex,
    fp8rl_quant_weight_blk128,
    fp8rl_quant_weight_blk128_batched,
    fp8rl_quant_weight_blk128_batched_ex,
    fp8rl_quant_weight_blk128_t,
    fp8rl_quant_weight_blk128_ex,
    fp8rl_scale_from_amax,
    WORKSPACE_HEADER_BYTES,
    SCRATCH_BYTES,
    quant_descs,
    tensor_descs,
    weight_descs,
    fp8rl_workspace_bytes,
    lib,
    new_workspace,
)

# Short aliases.
quant_weight = fp8rl_quant_weight_blk128
quant_weights = fp8rl_quant_weight_blk128_batched
quant_act = fp8rl_quant_act_tok128
gemm = fp8rl_gemm_w8a8_blockscaled
gemm_noalloc = fp8rl_gemm_w8a8_blockscaled_noalloc
gemm_fused_act = fp8rl_gemm_w8a8_fused_act_quant
grouped_gemm = fp8rl_grouped_gemm_w8a8
grouped_gemm_fused_act = fp8rl_grouped_gemm_w8a8_fused_act_quant
encode_e4m3 = fp8rl_encode_e4m3_f32
amax = fp8rl_amax_bf16
amax_batched = fp8rl_amax_bf16_batched
scale_from_amax = fp8rl_scale_from_amax
quant_per_tensor = fp8rl_quant_bf16_per_tensor
quant_per_tensor_batched = fp8rl_quant_bf16_per_tensor_batched
quant_weight_t = fp8rl_quant_weight_blk128_t
quant_colwise = fp8rl_quant_act_colwise128
gemm_rowscaled = fp8rl_gemm_w8a8_rowscaled
