// Host-side launchers behind the C ABI (arguments are validated before these are called).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8rl {

hipError_t launch_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w, uint8_t* wq,
                               int64_t ld_wq, float* sw, hipStream_t stream);
hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* xq,
                            int64_t ld_xq, float* sa, hipStream_t stream);
hipError_t launch_encode(const float* v, int64_t n, uint8_t* out, hipStream_t stream);

// GEMM planning: which tile configuration and how many K splits a shape uses. Pure host logic,
// shared by the workspace query and the launcher so both always agree.
struct GemmPlan {
  int cfg;     // tile configuration id (see gemm.hip)
  int bm, bn;  // workgroup tile
  int splits;  // K splits (1 = no split, result written directly)
  int kb_per_split;
  size_t workspace_bytes;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);
GemmPlan plan_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t E);

hipError_t launch_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, void* y, int out_f32, int64_t ld_y,
                       bool precise, void* workspace, const GemmPlan& plan, hipStream_t stream);
hipError_t launch_grouped_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq,
                               const float* sw, const int32_t* offsets, int32_t E,
                               int64_t M_total, int64_t N, int64_t K, void* y, int out_f32,
                               bool precise, void* workspace, const GemmPlan& plan,
                               hipStream_t stream);

}  // namespace fp8rl
