// Device helpers shared by the quantizer and GEMM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8rl {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 128;       // scale granularity along K (and along N for weights)
constexpr float kE4M3Max = 448.f; // largest finite E4M3 magnitude

// Widen the two bf16 values packed in a 32-bit word to float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |bf16| bit patterns of both halves (clears the two sign bits). For finite values the integer
// order of these patterns is the order of the magnitudes.
__device__ __forceinline__ uint32_t abs2_bf16(uint32_t w) { return w & 0x7FFF7FFFu; }

// Lane-wise max of two packed pairs of unsigned 16-bit values (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
  u16x2 r = __builtin_elementwise_max(x, y);
  return __builtin_bit_cast(uint32_t, r);
}

// Larger of the two 16-bit halves.
__device__ __forceinline__ uint32_t hmax_u16(uint32_t w) {
  uint32_t lo = w & 0xFFFFu, hi = w >> 16;
  return lo > hi ? lo : hi;
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15), result in every lane of the row.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2] and [2,3,0,1] reduce each quad; half-mirror joins quads 0-1 and 2-3;
  // mirror joins the two halves of the row.
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);
  v = v > t ? v : t;
  return v;
}

// Max over all 64 lanes of the wave, result in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  uint32_t t = (uint32_t)__shfl_xor((int)v, 16, 64);
  v = v > t ? v : t;
  t = (uint32_t)__shfl_xor((int)v, 32, 64);
  return v > t ? v : t;
}

// Scale of a group from the bit pattern of its largest |bf16| value:
//   S = fp32(amax / 448) (correctly rounded), or 1 when amax == 0.
// amax = X 2^a with X odd and < 2^8, and 448 = 7 2^6. A float32 rounding boundary m = M 2^c has
// an odd significand 2^24 <= M < 2^25; amax/448 == m would need X = 7M > 2^8, so it never
// happens, and |amax/448 - m| is a nonzero multiple of 2^min(a, c+6) / 448, i.e. at least about
// 2^-28 relative to m. The float64 product with RN64(1/448) is within 2^-51.9 of the exact
// quotient, so it sits on the same side of every boundary and rounds to RN32(amax / 448).
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bits16) {
  if (amax_bits16 == 0) return 1.0f;
  const double amax = (double)__uint_as_float(amax_bits16 << 16);
  return (float)(amax * (1.0 / 448.0));
}

// Power-of-two scale (the NeMo RL blog's power-of-2 scaling-factor option): the least 2^e with
// 448 * 2^e >= amax, e >= -127 (the smallest E8M0 value), 1 when amax == 0. With amax = f 2^E,
// f in [0.5, 1): 448 = 0.875 * 2^9, so e = E - 9 when f <= 0.875 and E - 8 otherwise; for a
// normal float32 amax with biased exponent ef and fraction bits t, E = ef - 126 and
// f > 0.875 <=> t > 0x600000. Exact: only exponent arithmetic.
__device__ __forceinline__ float pow2_scale_from_amax_bits(uint32_t amax_bits16) {
  if (amax_bits16 == 0) return 1.0f;
  const uint32_t a = amax_bits16 << 16;
  const int ef = (int)(a >> 23);
  int e = ef - 135 + ((a & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  if (ef == 0 || e < -127) e = -127;
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// E8M0 exponent byte of a power-of-two float32 scale (2^-127 .. 2^127): its biased exponent
// field (the subnormal 2^-127 has field 0, which is E8M0's 2^-127). The fraction bits of a scale
// that is not a power of two are ignored.
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xFFu); }

// Reciprocal of a (positive, finite, possibly subnormal) float32 scale, correctly rounded in
// float64. Used once per group/block; the element quotients are then formed as float64 products.
__device__ __forceinline__ double recip_f64(float s) { return 1.0 / (double)s; }

// IEEE float32 quotient x / S from the float64 reciprocal R = RN64(1/S).
//
// Exactness argument: x is a bf16 value (8 significant bits, odd part X < 2^8) and S a float32
// (odd part s < 2^24). A float32 rounding boundary (midpoint) m has an odd 25-bit significand M;
// x/S == m would need X == M * s, impossible since M >= 2^24 > X. Writing x = X 2^a, S = s 2^b,
// m = M 2^c, the difference x - mS is a nonzero multiple of 2^min(a, b+c), which bounds
// |x/S - m| / |m| below by about 2^-49. RN64(x * R) is within (1 + 2^-53)^2 - 1 < 2^-51.9 of
// x/S, so it lies on the same side of every float32 midpoint as x/S, and rounding it to float32
// (RNE) yields RN32(x / S). Quotients that fall in the float32 subnormal range are below 2^-126
// and all encode to a signed zero whichever way they round.
__device__ __forceinline__ float div_by_scale(float x, double r) { return (float)((double)x * r); }

// Clamp to the finite E4M3 range before conversion. For |t| <= 464 this does not change the
// nearest-even E4M3 code (448 is the nearest code to every value in (448, 464], ties at 464 go to
// the even mantissa of 448), and above it this is the saturation the format's encoder uses.
__device__ __forceinline__ float clamp_e4m3(float t) {
  return __builtin_amdgcn_fmed3f(t, -kE4M3Max, kE4M3Max);
}

// Pack four float32 values (already clamped) into four E4M3 bytes, v0 in the low byte.
// v_cvt_pk_fp8_f32 on gfx950 produces OCP E4M3 with round-to-nearest-even.
__device__ __forceinline__ uint32_t pack4_e4m3(float v0, float v1, float v2, float v3) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, r, true);
  return (uint32_t)r;
}

// Quantize the 8 bf16 values of one 16-byte chunk with reciprocal scale r; returns 8 codes.
__device__ __forceinline__ u32x2 quant8(u32x4 w, double r) {
  float f0 = clamp_e4m3(div_by_scale(bf16_lo(w.x), r));
  float f1 = clamp_e4m3(div_by_scale(bf16_hi(w.x), r));
  float f2 = clamp_e4m3(div_by_scale(bf16_lo(w.y), r));
  float f3 = clamp_e4m3(div_by_scale(bf16_hi(w.y), r));
  float f4 = clamp_e4m3(div_by_scale(bf16_lo(w.z), r));
  float f5 = clamp_e4m3(div_by_scale(bf16_hi(w.z), r));
  float f6 = clamp_e4m3(div_by_scale(bf16_lo(w.w), r));
  float f7 = clamp_e4m3(div_by_scale(bf16_hi(w.w), r));
  return u32x2{pack4_e4m3(f0, f1, f2, f3), pack4_e4m3(f4, f5, f6, f7)};
}

// Max |bf16| bit pattern over a 16-byte chunk, as packed 16-bit pairs.
__device__ __forceinline__ uint32_t amax8_pk(u32x4 w) {
  uint32_t a = pk_max_u16(abs2_bf16(w.x), abs2_bf16(w.y));
  uint32_t b = pk_max_u16(abs2_bf16(w.z), abs2_bf16(w.w));
  return pk_max_u16(a, b);
}

// Round a float32 to bf16 (nearest, ties to even); finite inputs.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace fp8rl
