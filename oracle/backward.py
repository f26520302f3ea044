"""FP8 backward pass of the W8A8 linear layer (input and weight gradients). TEST INFRASTRUCTURE.

What the pages fix:

* NeMo RL FP8 blog, Table 1: output gradients are E4M3 in [1, 128] groups with FP32 scales, like
  the input activations; weights stay in [128, 128] blocks;
* Unified FP8 blog (FP8-TI), quick-read section and its Megatron mixed-granularity figure:
  training as well as rollouts run the linears in FP8 -- forward (FProp), input gradient (Dgrad)
  and weight gradient (Wgrad) -- with per-token quantization for activations and gradients and
  per-block quantization for weights; its limitations paragraph notes that the training engine
  keeps a transposed copy of each quantized weight for the backward pass.

For Y = X W^T (X [M][K], W [N][K], Y [M][N]) and the output gradient dY [M][N]:

  Dgrad  dX[m][k] = sum_n dY[m][n] W[n][k]   (contraction over N)
  Wgrad  dW[n][k] = sum_m dY[m][n] X[m][k]   (contraction over the M tokens)

Readings where the pages leave a step open (each also listed in the design notes):

* B1 (Dgrad): dY is quantized in 1x128 groups along N (oracle.quant.quant_act_tok128); W uses its
  forward 128x128 blocks. A 128x128 block's amax does not depend on orientation, so the quantized
  W^T is the transpose of the quantized W (codes and block scales); Dgrad is the blockwise-scaled
  GEMM of dYq with that transposed copy.
* B2 (Wgrad): a per-token scale changes along the token axis, over which Wgrad sums, so it cannot
  be taken out of a 128-wide slice of that sum. Both operands are therefore quantized again in
  1x128 groups along the token axis -- i.e. the group quantizer applied to dY^T and X^T (128x1
  groups of dY and X) -- and Wgrad is the GEMM of dYq^T with Xq^T in which both operands carry one
  scale per row and 128-wide slice.
* B3: the token count M is a multiple of 128 for Wgrad (a caller pads with zero rows, which change
  neither an amax nor a sum).
"""

from __future__ import annotations

import numpy as np

from .gemm import _finish, dequant_act, gemm_blockscaled
from .quant import quant_act_tok128, quant_weight_blk128


def transpose_bits(bits) -> np.ndarray:
    """The transpose of a 2-D array (bf16 bit patterns, codes or scales), as a fresh C array."""
    return np.ascontiguousarray(np.asarray(bits).T)


def quant_weight_blk128_t(w_bits, scale: str = "fp32"):
    """B1: W^T quantized in 128x128 blocks: (WqT uint8 [K][N], swT float32 [K/128][N/128])."""
    return quant_weight_blk128(transpose_bits(w_bits), scale=scale)


def quant_colwise128(x_bits, scale: str = "fp32"):
    """B2: X [M][K] quantized in 128x1 groups (128 consecutive rows of one column), returned in
    the transposed layout: (XtQ uint8 [K][M], st float32 [K][M/128])."""
    return quant_act_tok128(transpose_bits(x_bits), scale=scale)


def gemm_rowscaled(aq, sa, bq, sb, out: str = "f64"):
    """Y[m][n] = sum_kb sa[m][kb] sb[n][kb] sum_{k in slice kb} dec(Aq[m][k]) dec(Bq[n][k]):
    both operands scaled per row and 128-wide K slice (B2). Both are dequantized like activations
    (exactly, in float64), multiplied in one float64 matmul and rounded once as `out` says."""
    A = dequant_act(aq, sa)
    B = dequant_act(bq, sb)
    if A.shape[1] != B.shape[1]:
        raise ValueError("K mismatch")
    return _finish(A @ B.T, out)


def linear_backward_fp8(dy_bits, x_bits, w_bits, out: str = "f64", scale: str = "fp32"):
    """dX and dW of Y = X W^T in FP8 (B1, B2): returns (dX [M][K], dW [N][K])."""
    dyq, s_dy = quant_act_tok128(dy_bits, scale=scale)
    wqt, swt = quant_weight_blk128_t(w_bits, scale=scale)
    dx = gemm_blockscaled(dyq, s_dy, wqt, swt, out=out)
    dytq, s_dyt = quant_colwise128(dy_bits, scale=scale)
    xtq, s_xt = quant_colwise128(x_bits, scale=scale)
    dw = gemm_rowscaled(dytq, s_dyt, xtq, s_xt, out=out)
    return dx, dw
