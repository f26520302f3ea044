/*
 * fp8rl.h -- C ABI of the MI355X (gfx950) FP8 blockwise-quantized W8A8 linear-layer library.
 *
 * The library implements the data-parallel hot path of an FP8 W8A8 linear layer as used for RL
 * rollouts with FP8 weights:
 *
 *   1. per-step re-quantization of bf16 weights W[N][K] to OCP E4M3 codes with one float32 scale
 *      per 128x128 block                      (fp8rl_quant_weight_blk128);
 *   2. dynamic per-token quantization of bf16 activations X[M][K] to E4M3 with one float32 scale
 *      per 1x128 group                         (fp8rl_quant_act_tok128);
 *   3. the blockwise-scaled FP8 GEMM Y = X W^T that consumes both
 *                                             (fp8rl_gemm_w8a8_blockscaled),
 *      and its mixture-of-experts grouped form (fp8rl_grouped_gemm_w8a8), and forms that
 *      take bf16 activations and quantize them themselves: inside the GEMM kernel for decode
 *      shapes (fp8rl_gemm_w8a8_fused_act_quant), once per token with the grouped GEMM reading
 *      the codes through the router's token indices (fp8rl_grouped_gemm_w8a8_fused_act_quant);
 *   plus the element-wise E4M3 encoder the quantizers share (fp8rl_encode_e4m3_f32), and the
 *   per-tensor FP8 of attention Q/K/V activations and the KV cache with per-step recalibrated
 *   scales (fp8rl_amax_bf16, fp8rl_scale_from_amax, fp8rl_quant_bf16_per_tensor and their
 *   batched forms).
 *
 * Sources, by page title and section:
 *   [UFP8]  "Unified FP8: Moving Beyond Mixed Precision for Stable and Accelerated MoE RL"
 *           (LMSYS blog digest), quick-read section: scale S = max|X| / V_max, Q(x) = round(x/S);
 *           "FP8 scale choice" section: FP32 scales rather than E8M0.
 *   [FP8RL] "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement Learning"
 *           (write-up), section 1 "dynamic weight sync": weights re-quantized after every update
 *           in independent 128x128 blocks, activations quantized dynamically, E4M3 with 4 exponent
 *           bits, 3 mantissa bits and range [-448, 448]; attention/MLP/MoE-expert linears in FP8.
 *   [NEMO]  NVIDIA NeMo RL FP8 blog, "FP8 for linear layers in RL", Table 1: weights E4M3 in
 *           [128,128] blocks, input activations E4M3 in [1,128] groups, FP32 block scales; FP8
 *           math for the linear layers. Section on FP8 for the KV cache and attention, Table 3:
 *           per-tensor FP32 scales for Q/K/V and the KV cache, recalibrated every step.
 *
 * Conventions for every entry point
 *   - Every pointer is a DEVICE pointer (memory the caller allocated on the current HIP device),
 *     except where marked "host". The library never allocates, frees or copies memory and never
 *     synchronizes: each call validates its arguments on the host, enqueues its kernel(s) on
 *     `stream` (a hipStream_t, passed as void* so that this header needs no HIP include; NULL
 *     means the default stream) and returns an fp8rl_status. Arguments that select an option
 *     (y_dtype, accum, scale_fmt, op) take the values of fp8rl_out_dtype, fp8rl_accum,
 *     fp8rl_scale_fmt and fp8rl_op as int; an unknown value is an error status, never a crash.
 *   - bf16 tensors are passed as uint16_t bit patterns; E4M3 codes as uint8_t (OCP E4M3: sign,
 *     4-bit exponent with bias 7, 3-bit mantissa, subnormals, no infinities, NaN = 0x7F/0xFF).
 *   - Row-major layouts; ld_* is the distance in ELEMENTS between consecutive rows.
 *   - Alignment: every base pointer must be 16-byte aligned (float scale arrays: 4-byte) and every
 *     row pitch in bytes (ld_* times the element size) a multiple of 16.
 *   - Shapes: K % 128 == 0, and N % 128 == 0 for weights and GEMMs; M >= 0 is arbitrary.
 *     A call with nothing to do (M == 0, or N == 0 / K == 0 for the weight quantizer) returns
 *     FP8RL_OK without touching memory or the stream. Dimensions must be below 2^31.
 *   - Errors: all validation happens before any HIP call; a failing check returns its status and
 *     enqueues nothing. FP8RL_ERR_HIP reports a failed launch. Faults inside a kernel surface at
 *     the caller's next synchronization. Inputs are read-only, outputs are fully overwritten
 *     (no bias, no accumulation into Y); outputs must not alias inputs.
 *   - Calls are re-entrant and may be made concurrently on different streams.
 */
#ifndef FP8RL_H
#define FP8RL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8RL_OK = 0,
  FP8RL_ERR_NULL = 1,      /* a required pointer is NULL */
  FP8RL_ERR_SHAPE = 2,     /* a dimension is negative, too large or not a multiple of 128 */
  FP8RL_ERR_ALIGN = 3,     /* a pointer or row pitch breaks the alignment rule */
  FP8RL_ERR_DTYPE = 4,     /* unknown output type */
  FP8RL_ERR_WORKSPACE = 5, /* workspace smaller than fp8rl_workspace_bytes() asks for */
  FP8RL_ERR_HIP = 6,       /* the HIP runtime rejected a launch */
  FP8RL_ERR_ARG = 7,       /* any other invalid argument (e.g. E < 1) */
  FP8RL_ERR_SCRATCH = 8    /* the shape needs more than FP8RL_SCRATCH_BYTES of GEMM scratch */
} fp8rl_status;

typedef enum { FP8RL_OUT_BF16 = 0, FP8RL_OUT_F32 = 1 } fp8rl_out_dtype;

typedef enum {
  FP8RL_OP_GEMM = 0,
  FP8RL_OP_GROUPED_GEMM = 1,
  FP8RL_OP_GEMM_ROWSCALED = 2,
  FP8RL_OP_GEMM_FUSED_ACT = 3,
  FP8RL_OP_GROUPED_GEMM_FUSED_ACT = 4
} fp8rl_op;

/*
 * How the matrix cores form the sum over one 128-wide K slice (the per-slice scaling, the float32
 * accumulation across slices and the final rounding are the same for all of them):
 *   FP8RL_ACCUM_FP8  the FP8 matrix-core instruction (v_mfma_f32_16x16x128_f8f6f4). Its internal
 *                    adder aligns the slice's products to the largest one and keeps about 15 bits
 *                    below it (measured on gfx950), comparable to the narrow FP8 accumulators the
 *                    Unified FP8 blog reports for Hopper tensor cores ("Tensor Core" hardware
 *                    table); promoting every 128-wide slice to float32 bounds the loss to one
 *                    slice. Full FP8 rate. Accepted with bf16 output only (FP8RL_ERR_ARG with
 *                    float32 output: its error is far above float32 rounding).
 *   FP8RL_ACCUM_F16  the same E4M3 codes widened exactly to f16 and summed by f16 matrix-core
 *                    instructions, whose adder keeps float32-level precision. Half the FP8 rate.
 *   FP8RL_ACCUM_MX   for power-of-two scales (FP8RL_SCALE_POW2): the block scales are applied by
 *                    the block-scaled FP8 matrix-core instruction (v_mfma_scale_f32_16x16x128_f8f6f4,
 *                    one E8M0 exponent per 32 K-values of a row; gfx950 has the E8M0 scaling units
 *                    the NeMo RL blog and the Unified FP8 blog say Hopper lacks), which also adds the
 *                    running float32 sum, so no per-slice float32 rescale is needed. Each slice sum
 *                    has the FP8 form's precision, so like FP8RL_ACCUM_FP8 it is accepted with
 *                    bf16 output only. Every sa and sw must be a power of two in [2^-127, 2^127]
 *                    (what the FP8RL_SCALE_POW2 quantizers produce); for any other scale value
 *                    the result is undefined (the scales are not inspected on the host, which
 *                    would need a synchronization). Shapes that run on the register-staged
 *                    64x64 tiles (17-1023 rows where the large DMA-fed tiles do not apply, an odd
 *                    K/128 at 17-64 rows, K > 32768) compute as FP8RL_ACCUM_FP8, which gives the
 *                    same results for power-of-two scales.
 *   FP8RL_ACCUM_AUTO the form that keeps the result within the library's accuracy contract
 *                    (elementwise |y - exact| <= 2^-7 |exact| + 1e-3 rms(exact) for bf16 output,
 *                    <= 1e-5 rms(exact) for float32 output, exact = the float64 sum over the
 *                    dequantized operands): FP8RL_ACCUM_FP8 for the blockscaled, fused and grouped
 *                    GEMMs with bf16 output; FP8RL_ACCUM_F16 for float32 output, and for the
 *                    row-scaled (weight-gradient) GEMM, whose long token sums can cancel far below
 *                    their slices' largest products. Never FP8RL_ACCUM_MX (ask for it).
 */
typedef enum {
  FP8RL_ACCUM_FP8 = 0,
  FP8RL_ACCUM_F16 = 1,
  FP8RL_ACCUM_MX = 2,
  FP8RL_ACCUM_AUTO = 3
} fp8rl_accum;

/*
 * Scale format of the quantizers (the _ex entry points):
 *   FP8RL_SCALE_FP32  S = fp32(amax / 448) [UFP8 quick-read; NEMO Table 1] -- the default.
 *   FP8RL_SCALE_POW2  S = the least power of two with 448 * S >= amax, at least 2^-127, 1 when
 *                     amax == 0 (the NeMo RL blog's advanced option that makes the weight and
 *                     activation scaling factors powers of 2 instead of FP32). Codes are then the
 *                     exact quotients x / S rounded onto the E4M3 grid; the scales are exact E8M0
 *                     values stored as float32.
 */
typedef enum { FP8RL_SCALE_FP32 = 0, FP8RL_SCALE_POW2 = 1 } fp8rl_scale_fmt;

/*
 * Element-wise E4M3 encoder: out[i] = nearest E4M3 code of v[i], ties to the even mantissa,
 * magnitudes above 448 saturate to +-448, the sign bit is always kept (so -0.0 and negative values
 * that round to zero give 0x80), NaN gives 0x7F with its sign.  This is the rounding step of
 * Q(x) = round(x / S) [UFP8, quick-read section] onto the E4M3 grid [FP8RL, section 1].
 *   v   : n float32 values (device, 16-byte aligned)
 *   out : n codes (device, 16-byte aligned)
 */
fp8rl_status fp8rl_encode_e4m3_f32(const float* v, int64_t n, uint8_t* out, void* stream);

/*
 * Weight re-quantization, 128x128 blocks [FP8RL, section 1; NEMO, Table 1; UFP8, quick-read].
 * For block (i, j) covering rows 128i..128i+127 and columns 128j..128j+127 of W[N][K]:
 *   amax      = max |W| over the block (exact on bf16),
 *   sw[i][j]  = fp32(amax / 448) by IEEE float32 division, or 1.0f when amax == 0,
 *   Wq[n][k]  = E4M3 code of fp32(W[n][k]) / sw[i][j] (IEEE float32 quotient, then the encoder
 *               above).
 *   w   : bf16 W, N rows of pitch ld_w (>= K) elements
 *   wq  : uint8 codes, N rows of pitch ld_wq (>= K)
 *   sw  : float32 scales, dense row-major [N/128][K/128]
 * Requires N % 128 == 0 and K % 128 == 0.
 */
fp8rl_status fp8rl_quant_weight_blk128(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                       uint8_t* wq, int64_t ld_wq, float* sw, void* stream);

/* The same with an explicit scale format (fp8rl_scale_fmt); FP8RL_ERR_ARG for an unknown one. */
fp8rl_status fp8rl_quant_weight_blk128_ex(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                          uint8_t* wq, int64_t ld_wq, float* sw, int scale_fmt,
                                          void* stream);

/* One weight matrix of a batched re-quantization (all pointers device, same rules as above). */
typedef struct {
  const uint16_t* w; /* bf16 W[N][ld_w] */
  uint8_t* wq;       /* uint8 Wq[N][ld_wq] */
  float* sw;         /* float32 sw[N/128][K/128] */
  int64_t N, K, ld_w, ld_wq;
} fp8rl_weight_desc;

/*
 * Batched weight re-quantization: the same operation as fp8rl_quant_weight_blk128 applied to
 * each of `count` matrices (e.g. every linear of a layer or a model, the per-step weight sync of
 * [FP8RL, section 1]), enqueued as ceil(count / 32) kernel launches instead of `count`.
 *   descs : HOST array of `count` descriptors; read during the call only.
 * Every descriptor is validated before anything is enqueued; the first failing one decides the
 * returned status and nothing is launched. Matrices with N == 0 or K == 0 are skipped.
 */
fp8rl_status fp8rl_quant_weight_blk128_batched(const fp8rl_weight_desc* descs, int32_t count,
                                               void* stream);

/* The same with an explicit scale format for every matrix (fp8rl_scale_fmt). */
fp8rl_status fp8rl_quant_weight_blk128_batched_ex(const fp8rl_weight_desc* descs, int32_t count,
                                                  int scale_fmt, void* stream);

/*
 * Dynamic activation quantization, 1x128 groups per token row [NEMO, Table 1; FP8RL, section 1;
 * UFP8, quick-read].  For row m and group g (columns 128g..128g+127 of X[M][K]):
 *   sa[m][g]  = fp32(max |X[m, group]| / 448), or 1.0f when that max is 0,
 *   Xq[m][k]  = E4M3 code of fp32(X[m][k]) / sa[m][k/128].
 *   x   : bf16 X, M rows of pitch ld_x (>= K)
 *   xq  : uint8 codes, M rows of pitch ld_xq (>= K)
 *   sa  : float32 scales, dense row-major [M][K/128]
 * Requires K % 128 == 0; any M >= 0.
 */
fp8rl_status fp8rl_quant_act_tok128(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                    uint8_t* xq, int64_t ld_xq, float* sa, void* stream);

/* The same with an explicit scale format (fp8rl_scale_fmt). */
fp8rl_status fp8rl_quant_act_tok128_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                       uint8_t* xq, int64_t ld_xq, float* sa, int scale_fmt,
                                       void* stream);

/*
 * Backward pass of the linear layer in FP8 [NEMO, Table 1: output gradients in [1,128] groups,
 * weights in [128,128] blocks, FP32 scales; UFP8, quick-read section and the Megatron
 * mixed-granularity figure: FProp, Dgrad and Wgrad in FP8 with per-token activations and
 * gradients and per-block weights; its limitations paragraph: a transposed copy of each quantized
 * weight is kept for the backward pass]. For Y = X W^T and the output gradient dY [M][N]:
 *   Dgrad  dX = dY W:     dYq, s_dy = fp8rl_quant_act_tok128(dY) (1x128 along N), then
 *                         fp8rl_gemm_w8a8_blockscaled(dYq, s_dy, WqT, swT) with M, N := K, K := N,
 *                         WqT / swT from fp8rl_quant_weight_blk128_t;
 *   Wgrad  dW = dY^T X:   dYtq, s_dyt = fp8rl_quant_act_colwise128(dY), Xtq, s_xt =
 *                         fp8rl_quant_act_colwise128(X) (128x1 groups along the tokens, stored
 *                         transposed), then fp8rl_gemm_w8a8_rowscaled(dYtq, s_dyt, Xtq, s_xt)
 *                         with M := N, N := K, K := tokens.
 * A per-token scale varies along Wgrad's summation axis, so Wgrad's operands are re-quantized in
 * groups along that axis; the token count must then be a multiple of 128 (pad with zero rows,
 * which change neither an amax nor a sum).
 */

/*
 * Weight quantization with a transposed copy: the 128x128 block quantization of W (as
 * fp8rl_quant_weight_blk128) and of W^T, which is its transpose (a block's amax does not depend
 * on orientation):  WqT[k][n] = Wq[n][k],  swT[k/128][n/128] = sw[n/128][k/128].
 *   wq, sw   : row-major codes [N][ld_wq] and scales [N/128][K/128], or both NULL (not written)
 *   wqt, swt : transposed codes [K][ld_wqt] (ld_wqt >= N) and scales [K/128][N/128]
 * Requires N % 128 == 0, K % 128 == 0; scale_fmt as for the _ex quantizers.
 */
fp8rl_status fp8rl_quant_weight_blk128_t(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                         uint8_t* wq, int64_t ld_wq, float* sw, uint8_t* wqt,
                                         int64_t ld_wqt, float* swt, int scale_fmt, void* stream);

/*
 * Column-group quantization with a transposed output (Wgrad operands): for column k of X[M][K]
 * and token group g (rows 128g .. 128g+127):
 *   sat[k][g]       = fp32(max |X[group, k]| / 448), or 1.0f when that max is 0,
 *   xtq[k][m]       = E4M3 code of fp32(X[m][k]) / sat[k][m/128]
 * i.e. fp8rl_quant_act_tok128 applied to X^T. Optionally (xq, sa not NULL) also the row-wise
 * 1x128 quantization of fp8rl_quant_act_tok128 from the same read of X (e.g. dY for Dgrad).
 *   xtq, sat : [K][ld_xtq] (ld_xtq >= M) codes and [K][M/128] scales
 *   xq, sa   : [M][ld_xq] codes and [M][K/128] scales, or both NULL
 * Requires M % 128 == 0 and K % 128 == 0; scale_fmt as for the _ex quantizers.
 */
fp8rl_status fp8rl_quant_act_colwise128(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                        uint8_t* xq, int64_t ld_xq, float* sa, uint8_t* xtq,
                                        int64_t ld_xtq, float* sat, int scale_fmt, void* stream);

/*
 * Blockwise-scaled W8A8 GEMM, Y = X W^T [NEMO, "FP8 for linear layers in RL"; FP8RL, section 1]:
 *   Y[m][n] = sum_kb sa[m][kb] * sw[n/128][kb] * sum_{k in slice kb} dec(Xq[m][k]) * dec(Wq[n][k])
 * with kb running over the K/128 slices of 128. Products of E4M3 values are exact; each slice's
 * sum is formed by the matrix cores as `accum` selects (fp8rl_accum), scaled in float32 by its
 * two block scales and added into a float32 accumulator; the result is rounded once (to nearest
 * even) to bf16 or kept as float32.
 *   xq, sa : activation codes [M][K] (pitch K) and scales [M][K/128]
 *   wq, sw : weight codes [N][K] (pitch K) and scales [N/128][K/128]
 *   y      : output [M][ld_y] (ld_y >= N) of type y_dtype
 *   accum  : FP8RL_ACCUM_AUTO (the form that meets the accuracy contract), FP8RL_ACCUM_FP8,
 *            FP8RL_ACCUM_F16 or FP8RL_ACCUM_MX (see fp8rl_accum); FP8 and MX with float32 output
 *            return FP8RL_ERR_ARG
 *   workspace, workspace_bytes: scratch of at least fp8rl_workspace_bytes(FP8RL_OP_GEMM, M, N, K, 0)
 *            bytes (device, 16-byte aligned; may be NULL when that size is 0). Its first
 *            FP8RL_WORKSPACE_HEADER_BYTES bytes hold arrival counters of the K-split reduction:
 *            they must be zero before the workspace is first used (allocate it zero-filled), and
 *            every call that returns FP8RL_OK leaves them zero again once its kernels have run,
 *            so one workspace serves any sequence of calls and shapes. Calls that use the same
 *            workspace must not run concurrently (different streams without ordering). The rest
 *            of the workspace is overwritten; the result does not depend on its contents.
 * Requires N % 128 == 0, K % 128 == 0. The result is deterministic (same bits every run).
 */
fp8rl_status fp8rl_gemm_w8a8_blockscaled(const uint8_t* xq, const float* sa, const uint8_t* wq,
                                         const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                         int y_dtype, int64_t ld_y, int accum, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * fp8rl_gemm_w8a8_blockscaled for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same operation,
 * kernels, results (the same bits) and argument rules, without the workspace arguments. The
 * scratch the call needs (K-split arrival counters and partials) is a static device array of
 * FP8RL_SCRATCH_BYTES that the library holds on every device it runs on until the process ends;
 * its first use on a device clears its counters (a small kernel on `stream`), and every call
 * leaves them zero again. A shape whose scratch need (fp8rl_workspace_bytes(FP8RL_OP_GEMM, M, N,
 * K, 0)) exceeds FP8RL_SCRATCH_BYTES returns FP8RL_ERR_SCRATCH without enqueuing anything.
 * The call never allocates or frees memory. All calls on one device share that device's array,
 * so calls that overlap on one GPU (different streams without ordering between them, or threads
 * enqueueing concurrently) race and give undefined results; order them on one stream.
 */
#define FP8RL_SCRATCH_BYTES (32u << 20)
fp8rl_status fp8rl_gemm_w8a8_blockscaled_noalloc(const uint8_t* xq, const float* sa,
                                                 const uint8_t* wq, const float* sw, int64_t M,
                                                 int64_t N, int64_t K, void* y, int y_dtype,
                                                 int64_t ld_y, int accum, void* stream);

/*
 * The blockwise-scaled GEMM on bf16 activations: quantize X in 1x128 groups and multiply, in one
 * call. [NEMO, speed-up discussion of the Llama 3 8B results: the quantization kernels placed
 * before each linear are overhead, and fusing them is expected to raise the gain further; UFP8,
 * limitations paragraph: at the small batches of RL the extra quantize steps leave the GPU
 * under-fed.] The result is bit-identical to fp8rl_quant_act_tok128_ex(x, scale_fmt) followed by
 * fp8rl_gemm_w8a8_blockscaled with the same accum. For M <= 4 it is one kernel: every workgroup
 * quantizes the activation slices it multiplies, so the FP8 activations never go to memory.
 * Above 4 rows that repeated quantization (every value once per 16- or 32-column tile) costs
 * more than the launch it saves, so the call stages the codes and scales in the workspace with
 * the 1x128 quantizer and runs the GEMM on them: two kernels, one call.
 *   x      : bf16 activations X, M rows of pitch ld_x (>= K; ld_x * 2 a multiple of 16)
 *   wq, sw, y, ld_y, accum : as for fp8rl_gemm_w8a8_blockscaled
 *   scale_fmt : FP8RL_SCALE_FP32 or FP8RL_SCALE_POW2, the activation groups' scale format;
 *            FP8RL_ACCUM_MX requires FP8RL_SCALE_POW2 (and power-of-two weight scales)
 *   workspace, workspace_bytes: at least fp8rl_workspace_bytes(FP8RL_OP_GEMM_FUSED_ACT, M, N, K,
 *            0) bytes (0 for M <= 4; above, the GEMM's own workspace followed by the staged
 *            codes and scales), 16-byte aligned, its first FP8RL_WORKSPACE_HEADER_BYTES zero
 *            before the first use (calls leave them zero)
 * Requires N % 128 == 0 and K % 128 == 0 (FP8RL_ERR_SHAPE otherwise; M == 0 returns FP8RL_OK).
 * Deterministic.
 */
fp8rl_status fp8rl_gemm_w8a8_fused_act_quant(const uint16_t* x, int64_t ld_x, const uint8_t* wq,
                                             const float* sw, int64_t M, int64_t N, int64_t K,
                                             void* y, int y_dtype, int64_t ld_y, int accum,
                                             int scale_fmt, void* workspace, size_t workspace_bytes,
                                             void* stream);

/*
 * Row-scaled FP8 GEMM (the weight-gradient product of the backward pass: both operands quantized
 * in 1x128 groups along the summed axis):
 *   Y[m][n] = sum_kb sa[m][kb] * sb[n][kb] * sum_{k in slice kb} dec(Aq[m][k]) * dec(Bq[n][k])
 * i.e. fp8rl_gemm_w8a8_blockscaled with one B scale per row and slice, sb [N][K/128], instead of
 * one per 128x128 block. Same arguments, rules, accumulation modes (with FP8RL_ACCUM_MX every sb
 * must be a power of two) and determinism. FP8RL_ACCUM_AUTO picks the f16 slice sums for both
 * output types here: a weight gradient sums thousands of tokens whose slices can cancel far below
 * their largest products, and the FP8 and MX forms' in-slice truncation (relative to that largest
 * product) can then exceed the bf16 tolerance; they stay available on request for bf16 output.
 * The workspace is sized by
 * fp8rl_workspace_bytes(FP8RL_OP_GEMM_ROWSCALED, M, N, K, 0).
 */
fp8rl_status fp8rl_gemm_w8a8_rowscaled(const uint8_t* aq, const float* sa, const uint8_t* bq,
                                       const float* sb, int64_t M, int64_t N, int64_t K, void* y,
                                       int y_dtype, int64_t ld_y, int accum, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Grouped (mixture-of-experts) blockwise-scaled W8A8 GEMM [FP8RL, section 1: MoE expert linears
 * are quantized like the other linears].  Rows off[e] .. off[e+1]-1 of Xq belong to expert e and
 * are multiplied by that expert's weights:
 *   Y[m][n] = sum_kb sa[m][kb] * sw[e][n/128][kb] * sum_k dec(Xq[m][k]) * dec(Wq[e][n][k])
 *   xq, sa           : [M_total][K] codes and [M_total][K/128] scales, rows grouped by expert
 *   wq, sw           : [E][N][K] codes and [E][N/128][K/128] scales
 *   expert_offsets   : E+1 int32 on the DEVICE; off[0] = 0, nondecreasing, off[E] = M_total
 *                      (read by the kernels, so no host synchronization is needed). Empty experts
 *                      are allowed. Row indices are clamped to [0, M_total], so a malformed array
 *                      cannot cause out-of-bounds accesses, but its result is then undefined.
 *   y                : [M_total][N] (pitch N), row order kept
 *   accum            : as for the dense GEMM (fp8rl_accum)
 *   workspace        : as for the dense GEMM, sized by fp8rl_workspace_bytes(FP8RL_OP_GROUPED_GEMM, ...)
 * Requires E >= 1, N % 128 == 0, K % 128 == 0.
 */
fp8rl_status fp8rl_grouped_gemm_w8a8(const uint8_t* xq, const float* sa, const uint8_t* wq,
                                     const float* sw, const int32_t* expert_offsets, int32_t E,
                                     int64_t M_total, int64_t N, int64_t K, void* y, int y_dtype,
                                     int accum, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * The grouped GEMM on bf16 activations: the activation quantization of
 * fp8rl_gemm_w8a8_fused_act_quant brought to the expert linears of a mixture-of-experts layer
 * [FP8RL, section 1: the MoE expert linears are quantized like the other linears; NEMO, speed-up
 * discussion of the Llama 3 8B results: the quantization kernels placed before the linears are
 * overhead]. Grouped row r (expert e owns rows expert_offsets[e] .. expert_offsets[e+1]-1, as in
 * fp8rl_grouped_gemm_w8a8) takes its activations from row row_ids[r] of x, the token the router
 * sent to that expert, so the caller passes the token activations as they are and the router's
 * token indices in expert order:
 *   Y[r][n] = sum_kb sa'[r][kb] * sw[e][n/128][kb]
 *             * sum_{k in slice kb} dec(Q(x[row_ids[r]])[k]) * dec(Wq[e][n][k])
 * with Q the 1x128 activation quantizer (scale format scale_fmt) and sa' its scales. The result
 * is bit-identical to fp8rl_quant_act_tok128_ex on the gathered rows x[row_ids[0 .. M_total-1]]
 * followed by fp8rl_grouped_gemm_w8a8 with the same accum: a 1x128 group lies within one row,
 * so a token quantized once has the same codes and scales for each expert it is sent to. Each
 * row of x is quantized once into the workspace (src_rows rows, against M_total = top-k x tokens
 * for the gathered form) and the grouped GEMM's tile DMA reads the codes and scales of the
 * listed rows, so no permuted copy of the activations is ever written. Two kernels in one call
 * (three where K > 32768: the grouped GEMM's register-staged tiles read contiguous rows, so a
 * copy kernel gathers the codes first).
 *   x          : bf16 activations, src_rows rows of pitch ld_x (>= K; ld_x * 2 a multiple of 16)
 *   src_rows   : rows of x; >= 1 when row_ids is given, and src_rows * K < 2^32
 *   row_ids    : M_total int32 on the DEVICE, or NULL. Each id is clamped to [0, src_rows - 1], so
 *                an out-of-range id reads the nearest valid row (never out of bounds). NULL: row r
 *                of x is grouped row r (src_rows must equal M_total), as for the down projection,
 *                whose input is already in expert order.
 *   wq, sw, expert_offsets, E, M_total, N, K, y, y_dtype, accum : as for fp8rl_grouped_gemm_w8a8
 *   scale_fmt  : FP8RL_SCALE_FP32 or FP8RL_SCALE_POW2 (FP8RL_ACCUM_MX requires FP8RL_SCALE_POW2)
 *   workspace, workspace_bytes : at least fp8rl_workspace_bytes(FP8RL_OP_GROUPED_GEMM_FUSED_ACT,
 *                max(src_rows, M_total), N, K, E) bytes, 16-byte aligned. The call does not touch
 *                its first FP8RL_WORKSPACE_HEADER_BYTES, so one workspace can serve this call and
 *                the dense GEMMs; the rest is overwritten.
 * Requires E >= 1, N % 128 == 0, K % 128 == 0 (FP8RL_ERR_SHAPE otherwise; M_total == 0 returns
 * FP8RL_OK). Deterministic.
 */
fp8rl_status fp8rl_grouped_gemm_w8a8_fused_act_quant(const uint16_t* x, int64_t ld_x,
                                                     int64_t src_rows, const int32_t* row_ids,
                                                     const uint8_t* wq, const float* sw,
                                                     const int32_t* expert_offsets, int32_t E,
                                                     int64_t M_total, int64_t N, int64_t K, void* y,
                                                     int y_dtype, int accum, int scale_fmt,
                                                     void* workspace, size_t workspace_bytes,
                                                     void* stream);

/*
 * Per-tensor FP8 for attention Q/K/V activations and the stored KV cache [NEMO, section on FP8
 * for the KV cache and attention, Table 3: E4M3 with one FP32 scale per tensor, the Q/K/V scales
 * recalibrated at the end of every training step from data run through the updated weights and
 * then handed to the inference engine; FP8RL, section 4 (KV-cache compression)]. Three calls:
 * accumulate each tensor's amax over its calibration batches, turn the amax values into scales,
 * and quantize new rows (into the KV cache) with a scale that stays in device memory.
 *
 * Shape rules for these calls (they differ from the 128-granular ones above): cols % 8 == 0,
 * ld_x >= cols with ld_x % 8 == 0, x 16-byte aligned, rows * cols / 8 < 2^31.
 */

/*
 * Running per-tensor amax: *amax = max(*amax, max |x|) over the bf16 tensor x[rows][ld_x]
 * (first `cols` elements of each row; exact). *amax must hold a non-negative float32 -- set it to
 * 0 before the first calibration batch -- and is updated with a device atomic, so calls on the
 * same amax may overlap. Values must be finite.
 *   x    : bf16 tensor, rows of pitch ld_x elements (e.g. the K columns of a fused QKV output)
 *   amax : one float32 (4-byte aligned)
 */
fp8rl_status fp8rl_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                             float* amax, void* stream);

/* One tensor of a batched amax (device pointers, rules as for fp8rl_amax_bf16). */
typedef struct {
  const uint16_t* x;
  float* amax;
  int64_t rows, cols, ld_x;
} fp8rl_tensor_desc;

/*
 * fp8rl_amax_bf16 for each of `count` tensors (e.g. Q, K and V of every layer), enqueued as
 * ceil(count / 32) launches. descs is a HOST array read during the call; every descriptor is
 * validated first and nothing is enqueued if one fails. Tensors with no elements are skipped.
 */
fp8rl_status fp8rl_amax_bf16_batched(const fp8rl_tensor_desc* descs, int32_t count, void* stream);

/*
 * Per-tensor scales from amax values: scale[i] = fp32(amax[i] / 448) by IEEE float32 division,
 * or 1.0f when amax[i] == 0 (the block quantizers' rule applied to a whole tensor).
 *   amax, scale : n float32 each (4-byte aligned; amax[i] non-negative and finite)
 */
fp8rl_status fp8rl_scale_from_amax(const float* amax, int32_t n, float* scale, void* stream);

/*
 * Per-tensor quantization of new rows, e.g. the K or V of new tokens into an FP8 KV cache:
 *   out[slot[r]][c] = E4M3 code of fp32(x[r][c]) / *scale   for r < rows, c < cols,
 * with the IEEE float32 quotient and the E4M3 encoder above (magnitudes beyond 448, i.e. values
 * larger than the calibrated amax, saturate to +-448). A row whose slot is negative or >= out_rows
 * is skipped (nothing written); with slot_mapping == NULL row r goes to out row r and rows <=
 * out_rows is required. Bytes of `out` outside the written rows and columns are untouched.
 *   x            : bf16 [rows][ld_x]
 *   scale        : one float32 on the device (positive, finite), e.g. from fp8rl_scale_from_amax
 *   out          : uint8 [out_rows][ld_out] (ld_out >= cols, ld_out % 8 == 0, 8-byte aligned)
 *   slot_mapping : `rows` int64 on the device (8-byte aligned), or NULL
 */
fp8rl_status fp8rl_quant_bf16_per_tensor(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ld_x, const float* scale, uint8_t* out,
                                         int64_t out_rows, int64_t ld_out,
                                         const int64_t* slot_mapping, void* stream);

/* One tensor of a batched per-tensor quantization (device pointers, rules as above). */
typedef struct {
  const uint16_t* x;
  const float* scale;
  uint8_t* out;
  const int64_t* slot_mapping; /* may be NULL */
  int64_t rows, cols, ld_x, out_rows, ld_out;
} fp8rl_quant_desc;

/*
 * fp8rl_quant_bf16_per_tensor for each of `count` tensors -- e.g. a layer's new K and V rows,
 * each with its own scale and cache -- enqueued as ceil(count / 16) launches. descs is a HOST
 * array read during the call; all descriptors are validated before anything is enqueued.
 * Outputs of different descriptors must not overlap.
 */
fp8rl_status fp8rl_quant_bf16_per_tensor_batched(const fp8rl_quant_desc* descs, int32_t count,
                                                 void* stream);

/* Bytes at the start of every GEMM workspace that hold the K-split arrival counters (see
 * fp8rl_gemm_w8a8_blockscaled). */
#define FP8RL_WORKSPACE_HEADER_BYTES 4096

/* Bytes of workspace the GEMM entry points need for this shape (0 when none; otherwise it includes
 * the FP8RL_WORKSPACE_HEADER_BYTES header). Host-only. */
size_t fp8rl_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int32_t E);

/* Static, NUL-terminated description of a status code. Host-only. */
const char* fp8rl_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. Host-only. */
int fp8rl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8RL_H */
