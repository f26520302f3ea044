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
  int block_begin[kWeightBatch];  // first grid block of matrix i (prefix sum of block counts)
  int count;
  int pow2;  // power-of-two scales instead of fp32(amax / 448)
};
hipError_t launch_quant_weight_batch(const WeightBatch& b, int total_blocks, hipStream_t stream);
hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* xq,
                            int64_t ld_xq, float* sa, int pow2, hipStream_t stream);
hipError_t launch_encode(const float* v, int64_t n, uint8_t* out, hipStream_t stream);

// GEMM planning: which tile configuration and how many K splits a shape uses. Pure host logic,
// shared by the workspace query and the launcher so both always agree.
struct GemmPlan {
  int cfg;     // tile configuration id (see gemm.hip)
  int bm, bn;  // workgroup tile
  int splits;  // K splits (1 = no split, result written directly)
  int kb_per_split;
  int depth;   // decode path: K slices in flight per wave
  size_t workspace_bytes;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);
GemmPlan plan_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t E);

hipError_t launch_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, void* y, int out_f32, int64_t ld_y,
                       int accum, void* workspace, const GemmPlan& plan, hipStream_t stream);
hipError_t launch_grouped_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq,
                               const float* sw, const int32_t* offsets, int32_t E,
                               int64_t M_total, int64_t N, int64_t K, void* y, int out_f32,
                               int accum, void* workspace, const GemmPlan& plan,
                               hipStream_t stream);

}  // namespace fp8rl
