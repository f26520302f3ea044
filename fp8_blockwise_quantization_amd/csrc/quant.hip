// Quantizer kernels: 128x128 weight blocks, 1x128 activation groups, element-wise E4M3 encode.
//
// Quantization rule (Unified FP8 blog, quick-read section; V_max = 448 and the E4M3 layout from
// the FP8-RL write-up, section 1; FP32 scales from the NeMo RL blog, Table 1):
//   S = fp32(amax / 448) (1 when amax == 0),  code = E4M3_RNE_sat(fp32(x) / S).
// With power-of-two scales (the NeMo RL blog's advanced FP8 options) S is instead the least power
// of two not below amax / 448 (at least 2^-127); the element step is the same.
// Both quotients are the IEEE float32 ones; see device_common.hpp for how they are formed exactly
// without a per-element division.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8rl {

// ---------------------------------------------------------------------------------------------
// Weights: one workgroup (4 waves) per 128x128 block. Thread t owns the 16-byte column chunk
// (t & 15) of rows (t >> 4) + 16 i, i = 0..7, so each load instruction of a wave reads four
// 256-byte row segments and the block (32 KiB of bf16) lives in registers between the amax pass
// and the encode pass: HBM traffic is one read of W and one write of Wq.
//
// One launch covers a batch of up to kWeightBatch matrices (a whole layer or model): the grid
// is the concatenation of every matrix's blocks, and each workgroup finds its matrix from the
// block prefix sums passed by value.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void quant_weight_block(const uint16_t* __restrict__ w, int64_t ld_w,
                                                   uint8_t* __restrict__ wq, int64_t ld_wq,
                                                   float* __restrict__ sw_out, int bi, int bj,
                                                   int pow2) {
  const int t = threadIdx.x;
  const int c = t & 15;
  const int r0 = t >> 4;

  const uint16_t* src = w + (int64_t)(bi * kBlock + r0) * ld_w + bj * kBlock + c * 8;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(16 * i) * ld_w));

  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = pk_max_u16(m, amax8_pk(v[i]));
  m = wave_max_u32(hmax_u16(m));

  __shared__ uint32_t red[4];
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = red[0];
  m = m > red[1] ? m : red[1];
  m = m > red[2] ? m : red[2];
  m = m > red[3] ? m : red[3];

  const float S = pow2 ? pow2_scale_from_amax_bits(m) : scale_from_amax_bits(m);
  const double r = recip_f64(S);
  if (t == 0) *sw_out = S;

  uint8_t* dst = wq + (int64_t)(bi * kBlock + r0) * ld_wq + bj * kBlock + c * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_nontemporal_store(quant8(v[i], r), reinterpret_cast<u32x2*>(dst + (int64_t)(16 * i) * ld_wq));
}

__global__ __launch_bounds__(256) void quant_weight_blk128_kernel(WeightBatch b) {
  const int bid = blockIdx.x;
  int t = 0;
#pragma unroll 1
  while (t + 1 < b.count && bid >= b.block_begin[t + 1]) ++t;  // uniform: bid is uniform
  const int local = bid - b.block_begin[t];
  const int KB = b.kb[t];
  const int bi = local / KB, bj = local - (local / KB) * KB;
  quant_weight_block(b.w[t], b.ld_w[t], b.wq[t], b.ld_wq[t], b.sw[t] + local, bi, bj, b.pow2);
}

// ---------------------------------------------------------------------------------------------
// Activations: each 16-lane DPP row of a wave owns one 1x128 group (8 bf16 per lane, one 16-byte
// load), reduces its amax with four DPP steps and writes 128 codes plus one scale. A workgroup
// covers 16 groups per step and STEPS steps, with all loads issued before any reduction (4 steps
// for large inputs; 1 for small ones, which then spread over 4x more workgroups and CUs).
// Group g is (row g / KB, slice g % KB), so neighbouring rows of a wave read neighbouring slices.
// ---------------------------------------------------------------------------------------------
template <int STEPS>
__global__ __launch_bounds__(256) void quant_act_tok128_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ xq, int64_t ld_xq,
    float* __restrict__ sa, int KB, int64_t total_groups, int pow2) {
  const int lane16 = threadIdx.x & 15;
  const int64_t g0 = (int64_t)blockIdx.x * (16 * STEPS) + (threadIdx.x >> 4);

  u32x4 v[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int64_t g = g0 + 16 * s;
    v[s] = u32x4{0u, 0u, 0u, 0u};
    if (g < total_groups) {
      const int64_t row = g / KB, slice = g - (g / KB) * KB;
      v[s] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(x + row * ld_x + slice * kBlock + lane16 * 8));
    }
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int64_t g = g0 + 16 * s;
    // every lane of the row takes part in the reduction, whether or not its group exists
    const uint32_t m = row16_max_u32(hmax_u16(amax8_pk(v[s])));
    const float S = pow2 ? pow2_scale_from_amax_bits(m) : scale_from_amax_bits(m);
    const double r = recip_f64(S);
    if (g < total_groups) {
      const int64_t row = g / KB, slice = g - (g / KB) * KB;
      if (lane16 == 0) sa[g] = S;
      __builtin_nontemporal_store(
          quant8(v[s], r), reinterpret_cast<u32x2*>(xq + row * ld_xq + slice * kBlock + lane16 * 8));
    }
  }
}

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
// Element-wise encoder (4 values per thread). NaN keeps its sign and becomes 0x7F; everything
// else is clamped to +-448 and converted with round-to-nearest-even.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float encode_prep(float f) {
  return __builtin_isnan(f) ? f : clamp_e4m3(f);
}

__device__ __forceinline__ uint32_t encode_fix_nan(uint32_t codes, float f, int byte) {
  if (__builtin_isnan(f)) {
    const uint32_t c = 0x7Fu | ((__float_as_uint(f) >> 24) & 0x80u);
    codes = (codes & ~(0xFFu << (8 * byte))) | (c << (8 * byte));
  }
  return codes;
}

__global__ __launch_bounds__(256) void encode_e4m3_kernel(const float* __restrict__ v, int64_t n,
                                                          uint8_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    const float4 f = *reinterpret_cast<const float4*>(v + i);
    uint32_t c = pack4_e4m3(encode_prep(f.x), encode_prep(f.y), encode_prep(f.z), encode_prep(f.w));
    c = encode_fix_nan(c, f.x, 0);
    c = encode_fix_nan(c, f.y, 1);
    c = encode_fix_nan(c, f.z, 2);
    c = encode_fix_nan(c, f.w, 3);
    *reinterpret_cast<uint32_t*>(out + i) = c;
  } else {
    for (int64_t j = i; j < n; ++j) {
      const float f = v[j];
      uint32_t c = pack4_e4m3(encode_prep(f), 0.f, 0.f, 0.f) & 0xFFu;
      c = encode_fix_nan(c, f, 0);
      out[j] = (uint8_t)c;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Launchers (arguments already validated by the C ABI layer).
// ---------------------------------------------------------------------------------------------
hipError_t launch_quant_weight_batch(const WeightBatch& b, int total_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(quant_weight_blk128_kernel, dim3((unsigned)total_blocks), dim3(256), 0, stream,
                     b);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* xq,
                            int64_t ld_xq, float* sa, int pow2, hipStream_t stream) {
  const int KB = (int)(K / kBlock);
  const int64_t groups = M * KB;
  if (groups >= int64_t{64} * 1024) {  // >= 1024 workgroups even at 4 steps each
    const int64_t wgs = (groups + 63) / 64;
    hipLaunchKernelGGL(quant_act_tok128_kernel<4>, dim3((unsigned)wgs), dim3(256), 0, stream, x,
                       ld_x, xq, ld_xq, sa, KB, groups, pow2);
  } else {
    const int64_t wgs = (groups + 15) / 16;
    hipLaunchKernelGGL(quant_act_tok128_kernel<1>, dim3((unsigned)wgs), dim3(256), 0, stream, x,
                       ld_x, xq, ld_xq, sa, KB, groups, pow2);
  }
  return hipGetLastError();
}

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

hipError_t launch_encode(const float* v, int64_t n, uint8_t* out, hipStream_t stream) {
  const int64_t threads = (n + 3) / 4;
  const int64_t wgs = (threads + 255) / 256;
  hipLaunchKernelGGL(encode_e4m3_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, v, n, out);
  return hipGetLastError();
}

}  // namespace fp8rl
