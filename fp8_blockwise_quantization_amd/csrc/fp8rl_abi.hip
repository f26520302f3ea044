// C ABI entry points: argument validation (host only, before any HIP call) and dispatch.
#include <stdint.h>

#include <algorithm>

#include "fp8rl.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fp8rl_status hip_status(hipError_t e) { return e == hipSuccess ? FP8RL_OK : FP8RL_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

fp8rl_status check_dims(int64_t a, int64_t b, int64_t c) {
  if (a < 0 || b < 0 || c < 0) return FP8RL_ERR_SHAPE;
  if (a > kMaxDim || b > kMaxDim || c > kMaxDim) return FP8RL_ERR_SHAPE;
  return FP8RL_OK;
}

// Shared checks of the dense and grouped GEMMs' operands.
fp8rl_status check_gemm_common(const uint8_t* xq, const float* sa, const uint8_t* wq,
                               const float* sw, int64_t N, int64_t K, const void* y, int y_dtype,
                               int64_t ld_y) {
  if (!xq || !sa || !wq || !sw || !y) return FP8RL_ERR_NULL;
  if (N == 0 || K == 0 || N % 128 || K % 128) return FP8RL_ERR_SHAPE;
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_DTYPE;
  if (ld_y < N) return FP8RL_ERR_SHAPE;
  const int64_t ybytes = y_dtype == FP8RL_OUT_F32 ? 4 : 2;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(sa, 4) ||
      !aligned(sw, 4) || (ld_y * ybytes) % 16)
    return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

// The accumulation form a GEMM call runs with, or -1 for an invalid request. FP8RL_ACCUM_AUTO
// resolves to the form that meets the accuracy contract (FP8 slice sums for bf16 output, f16 ones
// for float32 output and for every row-scaled call); the FP8 and MX forms are refused with float32
// output, whose tolerance their in-slice truncation does not meet.
int resolve_accum(int accum, int y_dtype, bool rowscaled) {
  if (accum == FP8RL_ACCUM_AUTO)
    return (y_dtype == FP8RL_OUT_F32 || rowscaled) ? FP8RL_ACCUM_F16 : FP8RL_ACCUM_FP8;
  if (accum != FP8RL_ACCUM_FP8 && accum != FP8RL_ACCUM_F16 && accum != FP8RL_ACCUM_MX) return -1;
  if (y_dtype == FP8RL_OUT_F32 && accum != FP8RL_ACCUM_F16) return -1;
  return accum;
}

}  // namespace

extern "C" {

int fp8rl_version(void) { return 200; }  // 0.2.0

const char* fp8rl_status_string(int s) {
  switch (s) {
    case FP8RL_OK: return "ok";
    case FP8RL_ERR_NULL: return "a required pointer is NULL";
    case FP8RL_ERR_SHAPE: return "invalid shape (negative, too large, or not a multiple of 128)";
    case FP8RL_ERR_ALIGN: return "pointer or row pitch not aligned as required";
    case FP8RL_ERR_DTYPE: return "unknown output dtype";
    case FP8RL_ERR_WORKSPACE: return "workspace too small";
    case FP8RL_ERR_HIP: return "HIP kernel launch failed";
    case FP8RL_ERR_ARG: return "invalid argument";
    case FP8RL_ERR_SCRATCH:
      return "shape needs more GEMM scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

fp8rl_status fp8rl_encode_e4m3_f32(const float* v, int64_t n, uint8_t* out, void* stream) {
  if (n < 0 || n > (int64_t{1} << 33)) return FP8RL_ERR_SHAPE;
  if (n == 0) return FP8RL_OK;
  if (!v || !out) return FP8RL_ERR_NULL;
  if (!aligned(v, 16) || !aligned(out, 16)) return FP8RL_ERR_ALIGN;
  return hip_status(fp8rl::launch_encode(v, n, out, as_stream(stream)));
}

namespace {

fp8rl_status check_weight(const fp8rl_weight_desc& d) {
  if (fp8rl_status s = check_dims(d.N, d.K, 0)) return s;
  if (d.N == 0 || d.K == 0) return FP8RL_OK;
  if (!d.w || !d.wq || !d.sw) return FP8RL_ERR_NULL;
  if (d.N % 128 || d.K % 128 || d.ld_w < d.K || d.ld_wq < d.K) return FP8RL_ERR_SHAPE;
  if ((d.N / 128) * (d.K / 128) >= (int64_t{1} << 24)) return FP8RL_ERR_SHAPE;  // grid limit
  if (!aligned(d.w, 16) || !aligned(d.wq, 16) || !aligned(d.sw, 4) || (d.ld_w * 2) % 16 ||
      d.ld_wq % 16)
    return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

// Launch the (already validated) descriptors in groups that fit one kernel's argument block
// and keep every grid below 2^24 workgroups.
fp8rl_status launch_weights(const fp8rl_weight_desc* descs, int32_t count, int pow2,
                            hipStream_t stream) {
  fp8rl::WeightBatch b{};
  b.pow2 = pow2;
  int64_t strips = 0;
  auto flush = [&]() -> fp8rl_status {
    if (b.count == 0) return FP8RL_OK;
    hipError_t e = fp8rl::launch_quant_weight_batch(b, (int)strips, stream);
    b = fp8rl::WeightBatch{};
    b.pow2 = pow2;
    strips = 0;
    return hip_status(e);
  };
  for (int32_t i = 0; i < count; ++i) {
    const fp8rl_weight_desc& d = descs[i];
    if (d.N == 0 || d.K == 0) continue;
    const int64_t nb = (d.N / 128) * ((d.K / 128 + 1) / 2);  // workgroups: 128x256 strips
    if (b.count == fp8rl::kWeightBatch || strips + nb >= (int64_t{1} << 24))
      if (fp8rl_status s = flush()) return s;
    b.w[b.count] = d.w;
    b.wq[b.count] = d.wq;
    b.sw[b.count] = d.sw;
    b.ld_w[b.count] = d.ld_w;
    b.ld_wq[b.count] = d.ld_wq;
    b.kb[b.count] = (int)(d.K / 128);
    b.block_begin[b.count] = (int)strips;
    ++b.count;
    strips += nb;
  }
  return flush();
}

}  // namespace

fp8rl_status fp8rl_quant_weight_blk128_ex(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                          uint8_t* wq, int64_t ld_wq, float* sw, int scale_fmt,
                                          void* stream) {
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  const fp8rl_weight_desc d{w, wq, sw, N, K, ld_w, ld_wq};
  if (fp8rl_status s = check_weight(d)) return s;
  return launch_weights(&d, 1, scale_fmt == FP8RL_SCALE_POW2, as_stream(stream));
}

fp8rl_status fp8rl_quant_weight_blk128(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                       uint8_t* wq, int64_t ld_wq, float* sw, void* stream) {
  return fp8rl_quant_weight_blk128_ex(w, N, K, ld_w, wq, ld_wq, sw, FP8RL_SCALE_FP32, stream);
}

fp8rl_status fp8rl_quant_weight_blk128_batched_ex(const fp8rl_weight_desc* descs, int32_t count,
                                                  int scale_fmt, void* stream) {
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (count < 0) return FP8RL_ERR_ARG;
  if (count == 0) return FP8RL_OK;
  if (!descs) return FP8RL_ERR_NULL;
  for (int32_t i = 0; i < count; ++i)
    if (fp8rl_status s = check_weight(descs[i])) return s;
  return launch_weights(descs, count, scale_fmt == FP8RL_SCALE_POW2, as_stream(stream));
}

fp8rl_status fp8rl_quant_weight_blk128_batched(const fp8rl_weight_desc* descs, int32_t count,
                                               void* stream) {
  return fp8rl_quant_weight_blk128_batched_ex(descs, count, FP8RL_SCALE_FP32, stream);
}

fp8rl_status fp8rl_quant_act_tok128_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                       uint8_t* xq, int64_t ld_xq, float* sa, int scale_fmt,
                                       void* stream) {
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (fp8rl_status s = check_dims(M, K, 0)) return s;
  if (M == 0 || K == 0) return FP8RL_OK;
  if (!x || !xq || !sa) return FP8RL_ERR_NULL;
  if (K % 128 || ld_x < K || ld_xq < K) return FP8RL_ERR_SHAPE;
  if (M * (K / 128) >= (int64_t{1} << 30)) return FP8RL_ERR_SHAPE;  // grid limit
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(sa, 4) || (ld_x * 2) % 16 || ld_xq % 16)
    return FP8RL_ERR_ALIGN;
  return hip_status(fp8rl::launch_quant_act(x, M, K, ld_x, xq, ld_xq, sa,
                                            scale_fmt == FP8RL_SCALE_POW2, as_stream(stream)));
}

fp8rl_status fp8rl_quant_act_tok128(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                    uint8_t* xq, int64_t ld_xq, float* sa, void* stream) {
  return fp8rl_quant_act_tok128_ex(x, M, K, ld_x, xq, ld_xq, sa, FP8RL_SCALE_FP32, stream);
}

namespace {

// Shape / alignment rules of the per-tensor calls; `empty` is set when there is nothing to do.
fp8rl_status check_tensor(const void* x, int64_t rows, int64_t cols, int64_t ld_x, bool& empty) {
  if (fp8rl_status s = check_dims(rows, cols, ld_x)) return s;
  empty = rows == 0 || cols == 0;
  if (empty) return FP8RL_OK;
  if (!x) return FP8RL_ERR_NULL;
  if (cols % 8 || ld_x < cols) return FP8RL_ERR_SHAPE;
  if (rows * (cols / 8) >= (int64_t{1} << 31)) return FP8RL_ERR_SHAPE;
  if (!aligned(x, 16) || ld_x % 8) return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

fp8rl_status check_amax_desc(const fp8rl_tensor_desc& d, bool& empty) {
  if (fp8rl_status s = check_tensor(d.x, d.rows, d.cols, d.ld_x, empty)) return s;
  if (empty) return FP8RL_OK;
  if (!d.amax) return FP8RL_ERR_NULL;
  if (!aligned(d.amax, 4)) return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

fp8rl_status launch_amax(const fp8rl_tensor_desc* descs, int32_t count, hipStream_t stream) {
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) total += descs[i].rows * (descs[i].cols / 8);
  const int launches = (count + fp8rl::kTensorBatch - 1) / fp8rl::kTensorBatch;
  const fp8rl::AmaxShape shape = fp8rl::amax_shape(total / launches);  // chunks of one launch
  const int64_t upw = int64_t{256} * shape.steps * shape.chunks;  // chunks per workgroup
  fp8rl::AmaxBatch b{};
  int64_t wgs = 0;
  auto reset = [&]() {
    b = fp8rl::AmaxBatch{};
    b.steps = shape.steps;
    b.chunks = shape.chunks;
    wgs = 0;
  };
  auto flush = [&]() -> fp8rl_status {
    if (b.count == 0) return FP8RL_OK;
    hipError_t e = fp8rl::launch_amax_batch(b, (int)wgs, stream);
    reset();
    return hip_status(e);
  };
  reset();
  for (int32_t i = 0; i < count; ++i) {
    const fp8rl_tensor_desc& d = descs[i];
    const int64_t units = d.rows * (d.cols / 8);
    if (units == 0) continue;
    const int64_t n = (units + upw - 1) / upw;
    if (b.count == fp8rl::kTensorBatch || wgs + n >= (int64_t{1} << 30))
      if (fp8rl_status s = flush()) return s;
    b.x[b.count] = d.x;
    b.amax[b.count] = d.amax;
    b.ld_x[b.count] = d.ld_x;
    b.cols8[b.count] = (int)(d.cols / 8);
    b.units[b.count] = (int)units;
    b.wg_begin[b.count] = (int)wgs;
    ++b.count;
    wgs += n;
  }
  return flush();
}

}  // namespace

fp8rl_status fp8rl_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                             float* amax, void* stream) {
  const fp8rl_tensor_desc d{x, amax, rows, cols, ld_x};
  bool empty = false;
  if (fp8rl_status s = check_amax_desc(d, empty)) return s;
  if (empty) return FP8RL_OK;
  return launch_amax(&d, 1, as_stream(stream));
}

fp8rl_status fp8rl_amax_bf16_batched(const fp8rl_tensor_desc* descs, int32_t count, void* stream) {
  if (count < 0) return FP8RL_ERR_ARG;
  if (count == 0) return FP8RL_OK;
  if (!descs) return FP8RL_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    bool empty = false;
    if (fp8rl_status s = check_amax_desc(descs[i], empty)) return s;
  }
  return launch_amax(descs, count, as_stream(stream));
}

fp8rl_status fp8rl_scale_from_amax(const float* amax, int32_t n, float* scale, void* stream) {
  if (n < 0) return FP8RL_ERR_SHAPE;
  if (n == 0) return FP8RL_OK;
  if (!amax || !scale) return FP8RL_ERR_NULL;
  if (!aligned(amax, 4) || !aligned(scale, 4)) return FP8RL_ERR_ALIGN;
  return hip_status(fp8rl::launch_scale_from_amax(amax, n, scale, as_stream(stream)));
}

namespace {

fp8rl_status check_quant_desc(const fp8rl_quant_desc& d, bool& empty) {
  if (fp8rl_status s = check_tensor(d.x, d.rows, d.cols, d.ld_x, empty)) return s;
  if (fp8rl_status s = check_dims(d.out_rows, d.ld_out, 0)) return s;
  if (empty) return FP8RL_OK;
  if (!d.scale || !d.out) return FP8RL_ERR_NULL;
  if (d.ld_out < d.cols || (!d.slot_mapping && d.rows > d.out_rows)) return FP8RL_ERR_SHAPE;
  if (!aligned(d.scale, 4) || !aligned(d.out, 8) || d.ld_out % 8 ||
      (d.slot_mapping && !aligned(d.slot_mapping, 8)))
    return FP8RL_ERR_ALIGN;
  return FP8RL_OK;
}

fp8rl_status launch_quant(const fp8rl_quant_desc* descs, int32_t count, hipStream_t stream) {
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) total += descs[i].rows * (descs[i].cols / 8);
  const int steps = fp8rl::quant_steps(total);
  const int64_t upw = int64_t{256} * steps;
  fp8rl::QuantBatch b{};
  int64_t wgs = 0;
  auto reset = [&]() {
    b = fp8rl::QuantBatch{};
    b.steps = steps;
    wgs = 0;
  };
  auto flush = [&]() -> fp8rl_status {
    if (b.count == 0) return FP8RL_OK;
    hipError_t e = fp8rl::launch_quant_batch(b, (int)wgs, stream);
    reset();
    return hip_status(e);
  };
  reset();
  for (int32_t i = 0; i < count; ++i) {
    const fp8rl_quant_desc& d = descs[i];
    const int64_t units = d.rows * (d.cols / 8);
    if (units == 0) continue;
    const int64_t n = (units + upw - 1) / upw;
    if (b.count == fp8rl::kQuantBatch || wgs + n >= (int64_t{1} << 30))
      if (fp8rl_status s = flush()) return s;
    const int c = b.count;
    b.x[c] = d.x;
    b.scale[c] = d.scale;
    b.out[c] = d.out;
    b.slot[c] = d.slot_mapping;
    b.ld_x[c] = d.ld_x;
    b.out_rows[c] = d.out_rows;
    b.ld_out[c] = d.ld_out;
    b.cols8[c] = (int)(d.cols / 8);
    b.units[c] = (int)units;
    b.wg_begin[c] = (int)wgs;
    ++b.count;
    wgs += n;
  }
  return flush();
}

}  // namespace

fp8rl_status fp8rl_quant_bf16_per_tensor(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ld_x, const float* scale, uint8_t* out,
                                         int64_t out_rows, int64_t ld_out,
                                         const int64_t* slot_mapping, void* stream) {
  const fp8rl_quant_desc d{x, scale, out, slot_mapping, rows, cols, ld_x, out_rows, ld_out};
  bool empty = false;
  if (fp8rl_status s = check_quant_desc(d, empty)) return s;
  if (empty) return FP8RL_OK;
  return launch_quant(&d, 1, as_stream(stream));
}

fp8rl_status fp8rl_quant_bf16_per_tensor_batched(const fp8rl_quant_desc* descs, int32_t count,
                                                 void* stream) {
  if (count < 0) return FP8RL_ERR_ARG;
  if (count == 0) return FP8RL_OK;
  if (!descs) return FP8RL_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    bool empty = false;
    if (fp8rl_status s = check_quant_desc(descs[i], empty)) return s;
  }
  return launch_quant(descs, count, as_stream(stream));
}

fp8rl_status fp8rl_quant_weight_blk128_t(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                         uint8_t* wq, int64_t ld_wq, float* sw, uint8_t* wqt,
                                         int64_t ld_wqt, float* swt, int scale_fmt, void* stream) {
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (fp8rl_status s = check_dims(N, K, 0)) return s;
  if (N == 0 || K == 0) return FP8RL_OK;
  if (!w || !wqt || !swt || (!wq) != (!sw)) return FP8RL_ERR_NULL;
  if (N % 128 || K % 128 || ld_w < K || ld_wqt < N || (wq && ld_wq < K)) return FP8RL_ERR_SHAPE;
  if ((N / 128) * (K / 128) >= (int64_t{1} << 24)) return FP8RL_ERR_SHAPE;  // grid limit
  if (!aligned(w, 16) || !aligned(wqt, 16) || !aligned(swt, 4) || (ld_w * 2) % 16 || ld_wqt % 16 ||
      (wq && (!aligned(wq, 16) || !aligned(sw, 4) || ld_wq % 16)))
    return FP8RL_ERR_ALIGN;
  const fp8rl::TileQuantArgs a{w, ld_w, (int)N, (int)K, wq, ld_wq, sw, wqt, ld_wqt, swt,
                               scale_fmt == FP8RL_SCALE_POW2};
  return hip_status(fp8rl::launch_quant_tile_t(a, 0, as_stream(stream)));
}

fp8rl_status fp8rl_quant_act_colwise128(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                        uint8_t* xq, int64_t ld_xq, float* sa, uint8_t* xtq,
                                        int64_t ld_xtq, float* sat, int scale_fmt, void* stream) {
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (fp8rl_status s = check_dims(M, K, 0)) return s;
  if (M == 0 || K == 0) return FP8RL_OK;
  if (!x || !xtq || !sat || (!xq) != (!sa)) return FP8RL_ERR_NULL;
  if (M % 128 || K % 128 || ld_x < K || ld_xtq < M || (xq && ld_xq < K)) return FP8RL_ERR_SHAPE;
  if ((M / 128) * (K / 128) >= (int64_t{1} << 24)) return FP8RL_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xtq, 16) || !aligned(sat, 4) || (ld_x * 2) % 16 || ld_xtq % 16 ||
      (xq && (!aligned(xq, 16) || !aligned(sa, 4) || ld_xq % 16)))
    return FP8RL_ERR_ALIGN;
  const fp8rl::TileQuantArgs a{x, ld_x, (int)M, (int)K, xq, ld_xq, sa, xtq, ld_xtq, sat,
                               scale_fmt == FP8RL_SCALE_POW2};
  return hip_status(fp8rl::launch_quant_tile_t(a, 1, as_stream(stream)));
}

size_t fp8rl_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int32_t E) {
  if (M <= 0 || N <= 0 || K <= 0 || N % 128 || K % 128) return 0;
  if (op == FP8RL_OP_GEMM) return fp8rl::plan_gemm(M, N, K).workspace_bytes;
  if (op == FP8RL_OP_GEMM_ROWSCALED) return fp8rl::plan_gemm(M, N, K, true).workspace_bytes;
  if (op == FP8RL_OP_GROUPED_GEMM) return fp8rl::plan_grouped_gemm(M, N, K, E).workspace_bytes;
  if (op == FP8RL_OP_GEMM_FUSED_ACT) return fp8rl::plan_fused_act(M, N, K).workspace_bytes;
  if (op == FP8RL_OP_GROUPED_GEMM_FUSED_ACT)
    return fp8rl::plan_grouped_fused_act(M, N, K, E).workspace_bytes;
  return 0;
}

namespace {

fp8rl_status gemm_common(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sw,
                         int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int64_t ld_y,
                         int accum, bool rowb, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (fp8rl_status s = check_dims(M, N, K)) return s;
  if (M == 0) return FP8RL_OK;
  if (fp8rl_status s = check_gemm_common(xq, sa, wq, sw, N, K, y, y_dtype, ld_y)) return s;
  accum = resolve_accum(accum, y_dtype, rowb);
  if (accum < 0) return FP8RL_ERR_ARG;
  if (((M + 127) / 128) * (N / 64) >= (int64_t{1} << 22)) return FP8RL_ERR_SHAPE;  // grid limit
  const fp8rl::GemmPlan plan = fp8rl::plan_gemm(M, N, K, rowb);
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return FP8RL_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8RL_ERR_ALIGN;
  }
  return hip_status(fp8rl::launch_gemm(xq, sa, wq, sw, M, N, K, y, y_dtype == FP8RL_OUT_F32, ld_y,
                                       accum, rowb, workspace, plan, as_stream(stream)));
}

}  // namespace

fp8rl_status fp8rl_gemm_w8a8_blockscaled(const uint8_t* xq, const float* sa, const uint8_t* wq,
                                         const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                         int y_dtype, int64_t ld_y, int accum, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return gemm_common(xq, sa, wq, sw, M, N, K, y, y_dtype, ld_y, accum, false, workspace,
                     workspace_bytes, stream);
}

fp8rl_status fp8rl_gemm_w8a8_blockscaled_noalloc(const uint8_t* xq, const float* sa,
                                                 const uint8_t* wq, const float* sw, int64_t M,
                                                 int64_t N, int64_t K, void* y, int y_dtype,
                                                 int64_t ld_y, int accum, void* stream) {
  if (fp8rl_status s = check_dims(M, N, K)) return s;
  if (M == 0) return FP8RL_OK;
  if (fp8rl_status s = check_gemm_common(xq, sa, wq, sw, N, K, y, y_dtype, ld_y)) return s;
  accum = resolve_accum(accum, y_dtype, false);
  if (accum < 0) return FP8RL_ERR_ARG;
  if (((M + 127) / 128) * (N / 64) >= (int64_t{1} << 22)) return FP8RL_ERR_SHAPE;
  const fp8rl::GemmPlan plan = fp8rl::plan_gemm(M, N, K, false);
  static_assert(fp8rl::kScratchBytes == FP8RL_SCRATCH_BYTES, "scratch size in the header");
  if (plan.workspace_bytes > fp8rl::kScratchBytes) return FP8RL_ERR_SCRATCH;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    if (fp8rl::gemm_scratch(as_stream(stream), &ws) != hipSuccess) return FP8RL_ERR_HIP;
  }
  return hip_status(fp8rl::launch_gemm(xq, sa, wq, sw, M, N, K, y, y_dtype == FP8RL_OUT_F32, ld_y,
                                       accum, false, ws, plan, as_stream(stream)));
}

fp8rl_status fp8rl_gemm_w8a8_fused_act_quant(const uint16_t* x, int64_t ld_x, const uint8_t* wq,
                                             const float* sw, int64_t M, int64_t N, int64_t K,
                                             void* y, int y_dtype, int64_t ld_y, int accum,
                                             int scale_fmt, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (fp8rl_status s = check_dims(M, N, K)) return s;
  if (M == 0) return FP8RL_OK;
  if (!x || !wq || !sw || !y) return FP8RL_ERR_NULL;
  if (N == 0 || K == 0 || N % 128 || K % 128) return FP8RL_ERR_SHAPE;
  if (ld_x < K || ld_x > kMaxDim) return FP8RL_ERR_SHAPE;
  if (M * (K / 128) >= (int64_t{1} << 30)) return FP8RL_ERR_SHAPE;                // quantizer grid
  if (((M + 127) / 128) * (N / 64) >= (int64_t{1} << 22)) return FP8RL_ERR_SHAPE;  // GEMM grid
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_DTYPE;
  if (ld_y < N) return FP8RL_ERR_SHAPE;
  accum = resolve_accum(accum, y_dtype, false);
  if (accum < 0) return FP8RL_ERR_ARG;
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (accum == FP8RL_ACCUM_MX && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  const int64_t ybytes = y_dtype == FP8RL_OUT_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ld_x * 2) % 16 || !aligned(wq, 16) || !aligned(sw, 4) ||
      !aligned(y, 16) || (ld_y * ybytes) % 16)
    return FP8RL_ERR_ALIGN;
  const fp8rl::GemmPlan plan = fp8rl::plan_fused_act(M, N, K);
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return FP8RL_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8RL_ERR_ALIGN;
  }
  return hip_status(fp8rl::launch_gemm_fused_act(
      x, ld_x, scale_fmt == FP8RL_SCALE_POW2, wq, sw, M, N, K, y, y_dtype == FP8RL_OUT_F32, ld_y,
      accum, workspace, plan, as_stream(stream)));
}

fp8rl_status fp8rl_gemm_w8a8_rowscaled(const uint8_t* aq, const float* sa, const uint8_t* bq,
                                       const float* sb, int64_t M, int64_t N, int64_t K, void* y,
                                       int y_dtype, int64_t ld_y, int accum, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return gemm_common(aq, sa, bq, sb, M, N, K, y, y_dtype, ld_y, accum, true, workspace,
                     workspace_bytes, stream);
}

fp8rl_status fp8rl_grouped_gemm_w8a8(const uint8_t* xq, const float* sa, const uint8_t* wq,
                                     const float* sw, const int32_t* expert_offsets, int32_t E,
                                     int64_t M_total, int64_t N, int64_t K, void* y, int y_dtype,
                                     int accum, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (fp8rl_status s = check_dims(M_total, N, K)) return s;
  if (E < 1 || E > 1024) return FP8RL_ERR_ARG;
  if (M_total == 0) return FP8RL_OK;
  if (!expert_offsets) return FP8RL_ERR_NULL;
  if (fp8rl_status s = check_gemm_common(xq, sa, wq, sw, N, K, y, y_dtype, N)) return s;
  accum = resolve_accum(accum, y_dtype, false);
  if (accum < 0) return FP8RL_ERR_ARG;
  if (!aligned(expert_offsets, 4)) return FP8RL_ERR_ALIGN;
  if (((M_total + 127) / 128 + E) * (N / 128) >= (int64_t{1} << 22)) return FP8RL_ERR_SHAPE;
  if ((int64_t)E * N * K >= (int64_t{1} << 40)) return FP8RL_ERR_SHAPE;
  const fp8rl::GemmPlan plan = fp8rl::plan_grouped_gemm(M_total, N, K, E);
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return FP8RL_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8RL_ERR_ALIGN;
  }
  return hip_status(fp8rl::launch_grouped_gemm(xq, sa, wq, sw, expert_offsets, E, M_total, N, K, y,
                                               y_dtype == FP8RL_OUT_F32, accum, workspace, plan,
                                               as_stream(stream)));
}

fp8rl_status fp8rl_grouped_gemm_w8a8_fused_act_quant(const uint16_t* x, int64_t ld_x,
                                                     int64_t src_rows, const int32_t* row_ids,
                                                     const uint8_t* wq, const float* sw,
                                                     const int32_t* expert_offsets, int32_t E,
                                                     int64_t M_total, int64_t N, int64_t K, void* y,
                                                     int y_dtype, int accum, int scale_fmt,
                                                     void* workspace, size_t workspace_bytes,
                                                     void* stream) {
  if (fp8rl_status s = check_dims(M_total, N, K)) return s;
  if (fp8rl_status s = check_dims(src_rows, ld_x, 0)) return s;
  if (E < 1 || E > 1024) return FP8RL_ERR_ARG;
  if (M_total == 0) return FP8RL_OK;
  if (!x || !wq || !sw || !y || !expert_offsets) return FP8RL_ERR_NULL;
  if (N == 0 || K == 0 || N % 128 || K % 128 || ld_x < K) return FP8RL_ERR_SHAPE;
  if (row_ids ? src_rows < 1 : src_rows != M_total) return FP8RL_ERR_SHAPE;
  if (row_ids && src_rows * K >= (int64_t{1} << 32)) return FP8RL_ERR_SHAPE;  // 32-bit DMA offsets
  if (src_rows * (K / 128) >= (int64_t{1} << 30)) return FP8RL_ERR_SHAPE;      // quantizer grid
  if (((M_total + 127) / 128 + E) * (N / 128) >= (int64_t{1} << 22)) return FP8RL_ERR_SHAPE;
  if ((int64_t)E * N * K >= (int64_t{1} << 40)) return FP8RL_ERR_SHAPE;
  if (y_dtype != FP8RL_OUT_BF16 && y_dtype != FP8RL_OUT_F32) return FP8RL_ERR_DTYPE;
  accum = resolve_accum(accum, y_dtype, false);
  if (accum < 0) return FP8RL_ERR_ARG;
  if (scale_fmt != FP8RL_SCALE_FP32 && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (accum == FP8RL_ACCUM_MX && scale_fmt != FP8RL_SCALE_POW2) return FP8RL_ERR_ARG;
  if (!aligned(x, 16) || (ld_x * 2) % 16 || !aligned(wq, 16) || !aligned(sw, 4) ||
      !aligned(y, 16) || !aligned(expert_offsets, 4) || (row_ids && !aligned(row_ids, 4)))
    return FP8RL_ERR_ALIGN;
  const fp8rl::GemmPlan plan =
      fp8rl::plan_grouped_fused_act(std::max(src_rows, M_total), N, K, E);
  if (!workspace || workspace_bytes < plan.workspace_bytes) return FP8RL_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FP8RL_ERR_ALIGN;
  return hip_status(fp8rl::launch_grouped_gemm_fused_act(
      x, ld_x, src_rows, row_ids, scale_fmt == FP8RL_SCALE_POW2, wq, sw, expert_offsets, E,
      M_total, N, K, y, y_dtype == FP8RL_OUT_F32, accum, workspace, as_stream(stream)));
}

}  // extern "C"
