// Quantizers with a transposed output, for the FP8 backward pass of the linear layer.
//
// Dgrad (dX = dY W) contracts over N, so it needs the weight codes laid out K-major: the 128x128
// block quantization of W^T, which is the transpose of W's (same blocks, same amax). Wgrad
// (dW = dY^T X) contracts over the tokens, so dY and X are quantized in 128x1 groups (128
// consecutive tokens of one column) and stored transposed, one 1x128 group per row of the output.
// (NeMo RL blog, Table 1: output gradients in [1,128] groups and weights in [128,128] blocks with
// FP32 scales; Unified FP8 blog: FProp, Dgrad and Wgrad in FP8 with per-token activations and
// gradients and per-block weights, and a transposed copy of each quantized weight kept for the
// backward pass.) The element rule is the forward one: code = E4M3_RNE_sat(fp32(x) / S).
//
// One workgroup (256 threads) per 128x128 tile of the bf16 input; thread t holds the 16-byte
// column chunk c = t & 15 of the 8 consecutive rows 8g .. 8g+7, g = t >> 4, so the tile sits in
// registers. Row-major codes, if asked for, are stored straight from registers. For the
// transposed codes a thread's 8 x 8 block of codes is transposed in registers (byte permutes),
// written to a 128 x 128-byte LDS tile as eight 8-byte pieces, and leaves as 16-byte row
// segments.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8rl {

constexpr int kTPitch = 144;  // bytes per LDS row of the transposed tile (128 codes + padding)

// Per-column amax of the tile (columns 8c .. 8c+7 of thread t's chunk c), as four packed pairs
// of 16-bit magnitudes, combined over the tile's 128 rows: in-thread over its 8 rows, across the
// four row groups of a wave that share c (lanes c + 16q), then across the four waves via LDS.
__device__ __forceinline__ void column_amax(const u32x4 (&v)[8], uint32_t (&red)[4][16][4],
                                            uint32_t (&cm)[4]) {
  const int t = threadIdx.x, c = t & 15, wave = t >> 6;
  cm[0] = cm[1] = cm[2] = cm[3] = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    cm[0] = pk_max_u16(cm[0], abs2_bf16(v[i].x));
    cm[1] = pk_max_u16(cm[1], abs2_bf16(v[i].y));
    cm[2] = pk_max_u16(cm[2], abs2_bf16(v[i].z));
    cm[3] = pk_max_u16(cm[3], abs2_bf16(v[i].w));
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    cm[p] = pk_max_u16(cm[p], (uint32_t)__shfl_xor((int)cm[p], 16, 64));
    cm[p] = pk_max_u16(cm[p], (uint32_t)__shfl_xor((int)cm[p], 32, 64));
  }
  if ((t & 63) < 16) {
#pragma unroll
    for (int p = 0; p < 4; ++p) red[wave][c][p] = cm[p];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p)
    cm[p] = pk_max_u16(pk_max_u16(red[0][c][p], red[1][c][p]), pk_max_u16(red[2][c][p], red[3][c][p]));
}

__device__ __forceinline__ float scale_of(uint32_t amax16, int pow2) {
  return pow2 ? pow2_scale_from_amax_bits(amax16) : scale_from_amax_bits(amax16);
}

// Codes of 8 values (one 16-byte chunk) with one reciprocal per value.
__device__ __forceinline__ u32x2 quant8_cols(u32x4 w, const double (&r)[8]) {
  float f0 = clamp_e4m3(div_by_scale(bf16_lo(w.x), r[0]));
  float f1 = clamp_e4m3(div_by_scale(bf16_hi(w.x), r[1]));
  float f2 = clamp_e4m3(div_by_scale(bf16_lo(w.y), r[2]));
  float f3 = clamp_e4m3(div_by_scale(bf16_hi(w.y), r[3]));
  float f4 = clamp_e4m3(div_by_scale(bf16_lo(w.z), r[4]));
  float f5 = clamp_e4m3(div_by_scale(bf16_hi(w.z), r[5]));
  float f6 = clamp_e4m3(div_by_scale(bf16_lo(w.w), r[6]));
  float f7 = clamp_e4m3(div_by_scale(bf16_hi(w.w), r[7]));
  return u32x2{pack4_e4m3(f0, f1, f2, f3), pack4_e4m3(f4, f5, f6, f7)};
}

// Byte e of each of 4 words, packed into one word (the word of `a0` in the low byte).
__device__ __forceinline__ uint32_t gather_byte(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                int e) {
  // v_perm_b32: selector byte k picks byte k' of {hi: first, lo: second}; 0x0c gives 0
  const uint32_t sel = 0x0c0c0000u | ((uint32_t)(4 + e) << 8) | (uint32_t)e;
  const uint32_t u = __builtin_amdgcn_perm(a1, a0, sel);  // [a0_e, a1_e, 0, 0]
  const uint32_t v = __builtin_amdgcn_perm(a3, a2, sel);  // [a2_e, a3_e, 0, 0]
  return __builtin_amdgcn_perm(v, u, 0x05040100u);          // [a0_e, a1_e, a2_e, a3_e]
}

// Transpose a thread's 8 x 8 codes (q[i]: row i, columns 0..7) and store column e's 8 codes (rows
// 0..7 in order) at transposed-tile row 8c + e, bytes row0 .. row0 + 7.
__device__ __forceinline__ void store_t(uint8_t* tq, const u32x2 (&q)[8], int c, int row0) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 2, b = e & 3;
    const uint32_t lo = gather_byte(q[0][w], q[1][w], q[2][w], q[3][w], b);
    const uint32_t hi = gather_byte(q[4][w], q[5][w], q[6][w], q[7][w], b);
    *reinterpret_cast<u32x2*>(tq + (8 * c + e) * kTPitch + row0) = u32x2{lo, hi};
  }
}

// ACT = 0: one scale for the whole tile (weights, 128x128 blocks); ACT = 1: one scale per column
// for the transposed codes (128x1 groups) and, for the optional row-major codes, one per row
// (1x128 groups, as the forward activation quantizer).
template <int ACT>
__global__ __launch_bounds__(256) void quant_tile_t_kernel(TileQuantArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tq[128 * kTPitch];
  __shared__ uint32_t red[4][16][4];
  const int tiles_c = a.C / kBlock, tiles_r = a.R / kBlock;
  const int bi = blockIdx.x / tiles_c, bj = blockIdx.x - (blockIdx.x / tiles_c) * tiles_c;
  const int t = threadIdx.x, c = t & 15, r0 = 8 * (t >> 4);  // rows r0 .. r0 + 7

  const uint16_t* src = a.x + (int64_t)(bi * kBlock + r0) * a.ld_x + bj * kBlock + c * 8;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)i * a.ld_x));
  u32x2 q[8];

  if constexpr (ACT == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = pk_max_u16(m, amax8_pk(v[i]));
    m = wave_max_u32(hmax_u16(m));
    if ((t & 63) == 0) red[t >> 6][0][0] = m;
    __syncthreads();
    m = red[0][0][0];
    m = m > red[1][0][0] ? m : red[1][0][0];
    m = m > red[2][0][0] ? m : red[2][0][0];
    m = m > red[3][0][0] ? m : red[3][0][0];
    const float S = scale_of(m, a.pow2);
    const double r = recip_f64(S);
    if (t == 0) {
      a.st[(int64_t)bj * tiles_r + bi] = S;
      if (a.s) a.s[(int64_t)bi * tiles_c + bj] = S;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      q[i] = quant8(v[i], r);
      if (a.q)
        __builtin_nontemporal_store(
            q[i], reinterpret_cast<u32x2*>(a.q + (int64_t)(bi * kBlock + r0 + i) * a.ld_q +
                                           bj * kBlock + c * 8));
    }
  } else {
    if (a.q) {  // row-major codes with 1x128 row groups
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t m = row16_max_u32(hmax_u16(amax8_pk(v[i])));
        const float S = scale_of(m, a.pow2);
        const int64_t row = (int64_t)bi * kBlock + r0 + i;
        if (c == 0) a.s[row * tiles_c + bj] = S;
        __builtin_nontemporal_store(
            quant8(v[i], recip_f64(S)),
            reinterpret_cast<u32x2*>(a.q + row * a.ld_q + bj * kBlock + c * 8));
      }
    }
    uint32_t cm[4];
    column_amax(v, red, cm);
    double r[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float s_lo = scale_of(cm[p] & 0xFFFFu, a.pow2);
      const float s_hi = scale_of(cm[p] >> 16, a.pow2);
      r[2 * p] = recip_f64(s_lo);
      r[2 * p + 1] = recip_f64(s_hi);
      if (t < 16) {
        const int64_t col = (int64_t)bj * kBlock + 8 * c + 2 * p;
        a.st[col * tiles_r + bi] = s_lo;
        a.st[(col + 1) * tiles_r + bi] = s_hi;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant8_cols(v[i], r);
  }
  store_t(tq, q, c, r0);
  __syncthreads();
  // transposed tile row j (source column bj*128 + j) holds the codes of source rows bi*128 ..
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int q = t + 256 * s, j = q >> 3, ch = q & 7;
    const u32x4 w = *reinterpret_cast<const u32x4*>(tq + j * kTPitch + ch * 16);
    __builtin_nontemporal_store(
        w, reinterpret_cast<u32x4*>(a.qt + (int64_t)(bj * kBlock + j) * a.ld_qt + bi * kBlock +
                                    ch * 16));
  }
}

hipError_t launch_quant_tile_t(const TileQuantArgs& a, int act, hipStream_t stream) {
  const unsigned tiles = (unsigned)((a.R / kBlock) * (a.C / kBlock));
  if (act)
    hipLaunchKernelGGL(quant_tile_t_kernel<1>, dim3(tiles), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(quant_tile_t_kernel<0>, dim3(tiles), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp8rl
