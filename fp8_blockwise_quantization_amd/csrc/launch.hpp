// Host-side launchers behind the C ABI (arguments are validated before these are called).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8rl {

// Up to kWeightBatch weight matrices quantized by one launch (passed by value as kernel
// arguments: 32 * 48 bytes + 4).
constexpr int kWeightBatch = 32;
struct WeightBatch {
  const uint16_t* w[kWeightBatch];
  uint8_t* wq[kWeightBatch];
  float* sw[kWeightBatch];
  int64_t ld_w[kWeightBatch];
  int64_t ld_wq[kWeightBatch];
  int kb[kWeightBatch];
  int block_begin[kWeightBatch];  // first workgroup of matrix i (prefix sum of its 128x256 strips)
  int count;
  int pow2;  // power-of-two scales instead of fp32(amax / 448)
};
hipError_t launch_quant_weight_batch(const WeightBatch& b, int total_strips, hipStream_t stream);
hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* xq,
                            int64_t ld_xq, float* sa, int pow2, hipStream_t stream);
hipError_t launch_encode(const float* v, int64_t n, uint8_t* out, hipStream_t stream);

// Per-tensor amax of up to kTensorBatch bf16 tensors in one launch (by value, like WeightBatch).
// A tensor is `units` 16-byte chunks (8 elements): chunk u is row u / cols8, column chunk
// u % cols8. Every workgroup reads steps * 256 * chunks consecutive chunks of one tensor.
constexpr int kTensorBatch = 32;
struct AmaxShape {
  int steps;   // chunks per thread per pass (1 or 8)
  int chunks;  // passes per workgroup
};
struct AmaxBatch {
  const uint16_t* x[kTensorBatch];
  float* amax[kTensorBatch];
  int64_t ld_x[kTensorBatch];
  int cols8[kTensorBatch];
  int units[kTensorBatch];
  int wg_begin[kTensorBatch];  // first workgroup of tensor i (prefix sum)
  int count;
  int steps, chunks;
};
AmaxShape amax_shape(int64_t total_units);
hipError_t launch_amax_batch(const AmaxBatch& b, int total_wgs, hipStream_t stream);
hipError_t launch_scale_from_amax(const float* amax, int n, float* scale, hipStream_t stream);
// Per-tensor quantization of up to kQuantBatch tensors in one launch (same chunk numbering as
// AmaxBatch; each workgroup covers 256 * steps chunks of one tensor).
constexpr int kQuantBatch = 16;
struct QuantBatch {
  const uint16_t* x[kQuantBatch];
  const float* scale[kQuantBatch];
  uint8_t* out[kQuantBatch];
  const int64_t* slot[kQuantBatch];
  int64_t ld_x[kQuantBatch];
  int64_t out_rows[kQuantBatch];
  int64_t ld_out[kQuantBatch];
  int cols8[kQuantBatch];
  int units[kQuantBatch];
  int wg_begin[kQuantBatch];
  int count;
  int steps;
};
int quant_steps(int64_t total_units);
hipError_t launch_quant_batch(const QuantBatch& b, int total_wgs, hipStream_t stream);

// Quantization of 128x128 tiles of a bf16 matrix X[R][C] with a transposed code output:
// qt [C][ld_qt] (and st) always, row-major q [R][ld_q] (and s) when q is not null.
// Weight mode: one scale per tile, s [R/128][C/128], st [C/128][R/128].
// Activation mode: st [C][R/128] per 128x1 column group; s [R][C/128] per 1x128 row group.
struct TileQuantArgs {
  const uint16_t* x;
  int64_t ld_x;
  int R, C;
  uint8_t* q;
  int64_t ld_q;
  float* s;
  uint8_t* qt;
  int64_t ld_qt;
  float* st;
  int pow2;
};
hipError_t launch_quant_tile_t(const TileQuantArgs& a, int act, hipStream_t stream);

// GEMM planning: which tile configuration and how many K splits a shape uses. Pure host logic,
// shared by the workspace query and the launcher so both always agree.
struct GemmPlan {
  int cfg;     // tile configuration id (see gemm.hip)
  int bm, bn;  // workgroup tile
  int splits;  // K splits (1 = no split, result written directly)
  int kb_per_split;
  int depth;   // streaming kernel: K slices in flight per wave; decode kernel: K halves per workgroup
  size_t workspace_bytes;
  size_t stage_off;  // fused activation quantization: workspace offset of the staged codes
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool rowb = false);
GemmPlan plan_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t E);

// rowb: sw is sb [N][K/128], one scale per row of B and K slice, instead of [N/128][K/128]
hipError_t launch_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, void* y, int out_f32, int64_t ld_y,
                       int accum, int rowb, void* workspace, const GemmPlan& plan,
                       hipStream_t stream);
// The library's own GEMM scratch for callers that cannot allocate: a static device array of
// kScratchBytes per device (see gemm.hip). Returns its address on the current device, clearing
// its counter header on the first use there (a fill kernel enqueued on `stream`).
constexpr size_t kScratchBytes = size_t{32} << 20;
hipError_t gemm_scratch(hipStream_t stream, void** ptr);
// The split-K decode GEMM's plan (5 <= M <= 64).
GemmPlan plan_decode(int64_t M, int64_t N, int64_t K);
// The GEMM with the 1x128 activation quantization fused in: bf16 X [M][ld_x] in place of xq / sa
// (pow2: scale format of the groups). Up to 4 rows one kernel quantizes in registers; above,
// the codes are staged in the workspace (from plan.stage_off) and the plan's GEMM reads them.
// Plans from plan_fused_act (its own workspace size).
GemmPlan plan_fused_act(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_fused_act(const uint16_t* x, int64_t ld_x, int pow2, const uint8_t* wq,
                                 const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                 int out_f32, int64_t ld_y, int accum, void* workspace,
                                 const GemmPlan& plan, hipStream_t stream);
// rows (device, M_total entries, or null): grouped row r reads the codes and scales of row
// rows[r] of xq / sa (clamped to [0, src_rows - 1]); DMA-fed tiles only (plan.cfg grouped-big),
// with src_rows * K < 2^32
hipError_t launch_grouped_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq,
                               const float* sw, const int32_t* offsets, int32_t E,
                               int64_t M_total, int64_t N, int64_t K, void* y, int out_f32,
                               int accum, void* workspace, const GemmPlan& plan,
                               hipStream_t stream, const int32_t* rows = nullptr,
                               int64_t src_rows = 0);
// The grouped GEMM on bf16 activations: x holds src_rows rows of pitch ld_x; grouped row r is
// row rows[r] (clamped), or row r when rows is null (then src_rows == M_total). Each source row
// is quantized once into the workspace (pow2: scale format), then the grouped GEMM gathers the
// codes through rows. The workspace is plan_grouped_fused_act(max(src_rows, M_total), N, K, E)'s.
GemmPlan plan_grouped_fused_act(int64_t M, int64_t N, int64_t K, int32_t E);
hipError_t launch_grouped_gemm_fused_act(const uint16_t* x, int64_t ld_x, int64_t src_rows,
                                         const int32_t* rows, int pow2, const uint8_t* wq,
                                         const float* sw, const int32_t* offsets, int32_t E,
                                         int64_t M_total, int64_t N, int64_t K, void* y,
                                         int out_f32, int accum, void* workspace,
                                         hipStream_t stream);

}  // namespace fp8rl
