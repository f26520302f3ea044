// Per-tensor FP8 kernels for attention Q/K/V activations and the stored KV cache.
//
// Rule (NeMo RL blog, section on FP8 for the KV cache and attention, Table 3: E4M3 with one FP32
// scale per tensor, recalibrated after every weight update; the scale and rounding rule of the
// Unified FP8 blog's quick-read section with V_max = 448):
//   S = fp32(amax / 448) (1 when amax == 0),  code = E4M3_RNE_sat(fp32(x) / S),
// the quotient formed exactly as in device_common.hpp.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8rl {

// ---------------------------------------------------------------------------------------------
// Per-tensor FP8 for attention Q/K/V activations and the stored KV cache (NeMo RL blog, section
// on the KV cache and attention, Table 3: one FP32 scale per tensor, recalibrated after every
// weight update from data run through the new weights). Three steps:
//   amax   -- running max|x| of each tensor over its calibration batches (one atomic max per
//             workgroup on the float bits, which order like the values for non-negative floats);
//   scale  -- S = fp32(amax / 448), 1 when amax == 0;
//   quant  -- codes of fp32(x) / S for new rows, written to cache row slot[r] (skipped when the
//             slot is negative or past the cache), the scale read from device memory so the
//             whole step runs without a host round trip.
// Work unit: a 16-byte chunk of 8 bf16; thread t of a workgroup takes chunks base + t + 256 s,
// s < STEPS, all loads issued before any use.
// ---------------------------------------------------------------------------------------------
template <int STEPS>
__global__ __launch_bounds__(256) void amax_bf16_kernel(AmaxBatch b) {
  const int bid = blockIdx.x;
  int t = 0;
#pragma unroll 1
  while (t + 1 < b.count && bid >= b.wg_begin[t + 1]) ++t;  // uniform: bid is uniform
  const uint16_t* __restrict__ x = b.x[t];
  const int64_t ld = b.ld_x[t];
  const unsigned cols8 = (unsigned)b.cols8[t], units = (unsigned)b.units[t];
  unsigned u0 = (unsigned)(bid - b.wg_begin[t]) * (256u * STEPS * b.chunks) + threadIdx.x;
  uint32_t m = 0;
#pragma unroll 1
  for (int ch = 0; ch < b.chunks; ++ch, u0 += 256u * STEPS) {
    u32x4 v[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const unsigned u = u0 + 256u * s;
      v[s] = u32x4{0u, 0u, 0u, 0u};
      if (u < units) {
        const unsigned row = u / cols8, c = u - row * cols8;
        v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + row * ld + c * 8));
      }
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) m = pk_max_u16(m, amax8_pk(v[s]));
  }
  m = wave_max_u32(hmax_u16(m));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = m > red[1] ? m : red[1];
    m = m > red[2] ? m : red[2];
    m = m > red[3] ? m : red[3];
    // The stored value only grows, so a workgroup whose max does not exceed what it reads has
    // nothing to add: most workgroups skip the (serializing, same-address) atomic.
    unsigned int* dst = reinterpret_cast<unsigned int*>(b.amax[t]);
    const unsigned cur = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((m << 16) > cur) atomicMax(dst, m << 16);
  }
}

__global__ __launch_bounds__(256) void scale_from_amax_kernel(const float* __restrict__ amax,
                                                              int n, float* __restrict__ scale) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float a = amax[i];
  scale[i] = a == 0.f ? 1.f : a / kE4M3Max;  // IEEE float32 division (correctly rounded)
}

template <int STEPS>
__global__ __launch_bounds__(256) void quant_per_tensor_kernel(QuantBatch b) {
  const int bid = blockIdx.x;
  int t = 0;
#pragma unroll 1
  while (t + 1 < b.count && bid >= b.wg_begin[t + 1]) ++t;  // uniform: bid is uniform
  const uint16_t* __restrict__ x = b.x[t];
  const int64_t* __restrict__ slot = b.slot[t];
  const int64_t ld_x = b.ld_x[t], ld_out = b.ld_out[t], out_rows = b.out_rows[t];
  const unsigned cols8 = (unsigned)b.cols8[t], units = (unsigned)b.units[t];
  const unsigned u0 = (unsigned)(bid - b.wg_begin[t]) * (256u * STEPS) + threadIdx.x;
  u32x4 v[STEPS];
  int64_t dst[STEPS];  // byte offset of the chunk's codes, or -1 when nothing is stored
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const unsigned u = u0 + 256u * s;
    v[s] = u32x4{0u, 0u, 0u, 0u};
    dst[s] = -1;
    if (u < units) {
      const unsigned row = u / cols8, c = u - row * cols8;
      v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + row * ld_x + c * 8));
      const int64_t orow = slot ? slot[row] : (int64_t)row;
      if (orow >= 0 && orow < out_rows) dst[s] = orow * ld_out + c * 8;
    }
  }
  const double r = recip_f64(*b.scale[t]);
  uint8_t* __restrict__ out = b.out[t];
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
    if (dst[s] >= 0)
      __builtin_nontemporal_store(quant8(v[s], r), reinterpret_cast<u32x2*>(out + dst[s]));
}

// ---------------------------------------------------------------------------------------------
// Launchers (arguments already validated by the C ABI layer).
// ---------------------------------------------------------------------------------------------
// Workgroup size of the amax pass in 16-byte chunks, from the chunks of one launch: 8 per thread
// and enough passes per workgroup that a large launch has about 512 workgroups, two per CU with
// 64 KiB of loads in flight each -- measured faster than 4x more, shorter workgroups (fewer
// same-address atomics, no tail); one chunk per thread for small inputs.
AmaxShape amax_shape(int64_t total_units) {
  if (total_units < (int64_t{2} << 20)) return AmaxShape{1, 1};
  const int64_t chunks = total_units / (int64_t{2048} * 512);
  return AmaxShape{8, (int)(chunks < 1 ? 1 : chunks > 256 ? 256 : chunks)};
}

hipError_t launch_amax_batch(const AmaxBatch& b, int total_wgs, hipStream_t stream) {
  if (b.steps == 8)
    hipLaunchKernelGGL(amax_bf16_kernel<8>, dim3((unsigned)total_wgs), dim3(256), 0, stream, b);
  else
    hipLaunchKernelGGL(amax_bf16_kernel<1>, dim3((unsigned)total_wgs), dim3(256), 0, stream, b);
  return hipGetLastError();
}

hipError_t launch_scale_from_amax(const float* amax, int n, float* scale, hipStream_t stream) {
  hipLaunchKernelGGL(scale_from_amax_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, amax, n, scale);
  return hipGetLastError();
}

// Chunks per thread of the per-tensor quantizer: about 2048 or more workgroups per launch (all
// of a mid-sized launch's loads in flight at once), up to 8 chunks per thread for large ones.
int quant_steps(int64_t total_units) {
  const int64_t per = total_units / (int64_t{2048} * 256);
  return per >= 8 ? 8 : per >= 4 ? 4 : per >= 2 ? 2 : 1;
}

hipError_t launch_quant_batch(const QuantBatch& b, int total_wgs, hipStream_t stream) {
  const dim3 g((unsigned)total_wgs), t(256);
  switch (b.steps) {
    case 8: hipLaunchKernelGGL(quant_per_tensor_kernel<8>, g, t, 0, stream, b); break;
    case 4: hipLaunchKernelGGL(quant_per_tensor_kernel<4>, g, t, 0, stream, b); break;
    case 2: hipLaunchKernelGGL(quant_per_tensor_kernel<2>, g, t, 0, stream, b); break;
    default: hipLaunchKernelGGL(quant_per_tensor_kernel<1>, g, t, 0, stream, b); break;
  }
  return hipGetLastError();
}

}  // namespace fp8rl
