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
// Weights: one workgroup (8 waves) per pair of horizontally adjacent 128x128 blocks, a 128x256
// strip of W (the last strip of a block row is a single block when K/128 is odd). Thread t owns
// the 16-byte column chunk c = t & 31 of rows (t >> 5) + 16 i, i = 0..7, so each load
// instruction of a wave reads two 512-byte row segments; chunks c < 16 lie in the left block,
// the others in the right one. The strip (64 KiB of bf16) stays in registers between the amax
// pass and the encode pass: HBM traffic is one read of W and one write of Wq. Measured on the
// Qwen3-8B block's 7 weights: whole 512-byte row segments stream faster than one block's 256-byte
// ones, and 8 waves per strip (8 loads per thread) beat 4 (16 loads, fewer resident waves) and
// 16 (4 loads, more barrier and reduction work per byte).
//
// One launch covers a batch of up to kWeightBatch matrices (a whole layer or model): the grid
// is the concatenation of every matrix's strips, and each workgroup finds its matrix from the
// strip prefix sums passed by value.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void quant_weight_pair(const uint16_t* __restrict__ w, int64_t ld_w,
                                                  uint8_t* __restrict__ wq, int64_t ld_wq,
                                                  float* __restrict__ sw_row, int bi, int bp,
                                                  int KB, int pow2) {
  const int t = threadIdx.x;
  const int c = t & 31, r0 = t >> 5;  // r0 < 16
  const int hb = c >> 4;               // 0: left block, 1: right block
  const int bj = 2 * bp + hb;          // this lane's block column
  const bool live = bj < KB;           // false only in the missing right block of an odd row

  const uint16_t* src = w + (int64_t)(bi * kBlock + r0) * ld_w + bp * (2 * kBlock) + c * 8;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (live)
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(16 * i) * ld_w));
  }

  // lane l of wave q holds row 2q + (l >> 5) of block (l >> 4) & 1: a DPP row (16 lanes) is one
  // block's 256-byte segment of one row, and lanes l and l ^ 32 belong to the same block
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = pk_max_u16(m, amax8_pk(v[i]));
  m = row16_max_u32(hmax_u16(m));
  const uint32_t o = (uint32_t)__shfl_xor((int)m, 32, 64);
  m = m > o ? m : o;

  __shared__ uint32_t red[2][8];
  const int lane = t & 63, wv = t >> 6;
  if (lane == 0) red[0][wv] = m;
  if (lane == 16) red[1][wv] = m;
  __syncthreads();
  m = red[hb][0];
#pragma unroll
  for (int k = 1; k < 8; ++k) m = m > red[hb][k] ? m : red[hb][k];
  if (!live) return;

  const float S = pow2 ? pow2_scale_from_amax_bits(m) : scale_from_amax_bits(m);
  const double r = recip_f64(S);
  if (t == 0 || t == 16) sw_row[bj] = S;

  uint8_t* dst = wq + (int64_t)(bi * kBlock + r0) * ld_wq + bp * (2 * kBlock) + c * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_nontemporal_store(quant8(v[i], r), reinterpret_cast<u32x2*>(dst + (int64_t)(16 * i) * ld_wq));
}

__global__ __launch_bounds__(512) void quant_weight_blk128_kernel(WeightBatch b) {
  const int bid = blockIdx.x;
  int t = 0;
#pragma unroll 1
  while (t + 1 < b.count && bid >= b.block_begin[t + 1]) ++t;  // uniform: bid is uniform
  const int local = bid - b.block_begin[t];
  const int KB = b.kb[t];
  const int KP = (KB + 1) >> 1;  // strips per block row
  const int bi = local / KP, bp = local - (local / KP) * KP;
  quant_weight_pair(b.w[t], b.ld_w[t], b.wq[t], b.ld_wq[t], b.sw[t] + (int64_t)bi * KB, bi, bp,
                    KB, b.pow2);
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
    float* __restrict__ sa, int KB, int total_groups, int pow2) {
  // group indices fit 32 bits (the C ABI keeps M * K/128 below 2^30): 32-bit division only
  const int lane16 = threadIdx.x & 15;
  const unsigned g0 = blockIdx.x * (16u * STEPS) + (threadIdx.x >> 4);
  const unsigned kb = (unsigned)KB, total = (unsigned)total_groups;

  u32x4 v[STEPS];
  int64_t xoff[STEPS], qoff[STEPS];  // element offsets of the group's 16-byte chunk in X and Xq
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const unsigned g = g0 + 16u * s;
    const unsigned row = g / kb, slice = g - row * kb;
    xoff[s] = (int64_t)row * ld_x + slice * kBlock + lane16 * 8;
    qoff[s] = (int64_t)row * ld_xq + slice * kBlock + lane16 * 8;
    v[s] = u32x4{0u, 0u, 0u, 0u};
    if (g < total) v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + xoff[s]));
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const unsigned g = g0 + 16u * s;
    // every lane of the row takes part in the reduction, whether or not its group exists
    const uint32_t m = row16_max_u32(hmax_u16(amax8_pk(v[s])));
    const float S = pow2 ? pow2_scale_from_amax_bits(m) : scale_from_amax_bits(m);
    const double r = recip_f64(S);
    if (g < total) {
      if (lane16 == 0) sa[g] = S;
      __builtin_nontemporal_store(quant8(v[s], r), reinterpret_cast<u32x2*>(xq + qoff[s]));
    }
  }
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
hipError_t launch_quant_weight_batch(const WeightBatch& b, int total_strips, hipStream_t stream) {
  hipLaunchKernelGGL(quant_weight_blk128_kernel, dim3((unsigned)total_strips), dim3(512), 0, stream,
                     b);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* xq,
                            int64_t ld_xq, float* sa, int pow2, hipStream_t stream) {
  const int KB = (int)(K / kBlock);
  const int64_t groups = M * KB;  // < 2^30 (checked by the C ABI)
  if (groups >= int64_t{64} * 1024) {  // >= 1024 workgroups even at 4 steps each
    const int64_t wgs = (groups + 63) / 64;
    hipLaunchKernelGGL(quant_act_tok128_kernel<4>, dim3((unsigned)wgs), dim3(256), 0, stream, x,
                       ld_x, xq, ld_xq, sa, KB, (int)groups, pow2);
  } else {
    const int64_t wgs = (groups + 15) / 16;
    hipLaunchKernelGGL(quant_act_tok128_kernel<1>, dim3((unsigned)wgs), dim3(256), 0, stream, x,
                       ld_x, xq, ld_xq, sa, KB, (int)groups, pow2);
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
