// Blockwise-scaled W8A8 GEMM and its grouped (MoE) form on gfx950 FP8 matrix cores.
//
//   Y[m][n] = sum_kb sa[m][kb] * sw[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum over the 128 k of slice kb of dec(Xq[m][k]) * dec(Wq[n][k])
//
// (NeMo RL blog, "FP8 for linear layers in RL", Table 1: [1,128] activation and [128,128] weight
// scales in FP32; FP8-RL write-up, section 1.) One K step of the kernel is exactly one 128-wide
// scale slice, and one v_mfma_f32_16x16x128_f8f6f4 covers it for a 16x16 output tile, so P_kb
// comes out of the matrix core as a float32 tile that is then scaled by sa*sw and added into a
// float32 accumulator with one FMA per element.
//
// Data flow per workgroup: Xq and Wq tiles of one K slice (BM x 128 and BN x 128 bytes) are
// copied global -> registers -> LDS with a double buffer (the next slice's global loads are in
// flight while the current slice is multiplied), the activation scales of the slice go to LDS
// beside them, and the weight scale of a wave's 128-column block is a wave-uniform load.
// LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk c ^ swz(r) with
// swz(r) = (r & 7) ^ ((r >> 3) & 1). A fragment read has 16 consecutive rows read the same
// logical chunk: any 8 consecutive rows then hit 8 different 16-byte bank groups of a 128-byte
// row, and the 8 even (odd) rows of 16 hit 8 different groups too, so the read is free of bank
// conflicts whether the LDS serves 8 lanes (32 banks) or 16 lanes (64 banks) per cycle.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8rl {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ROWB_: the B operand carries one scale per row and K slice (sb[N][KB]) instead of one per
// 128x128 block; those scales then travel with each slice like the activation scales.
template <int BM_, int BN_, int WM_, int WN_, bool ROWB_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool ROWB = ROWB_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int NT = WAVES * 64;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + BM * 4 + (ROWB ? BN * 4 : 0);
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int A_LOADS = BM * 8 / NT;
  static constexpr int B_LOADS = BN * 8 / NT;
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile must split into 16-byte loads");
  static_assert(BM <= NT && BN <= NT, "one scale load per tile row");
  static_assert(128 % WN == 0, "a wave's columns must share one weight-scale block");
};

using TileLarge = Tile<128, 128, 64, 64>;  // prefill-sized M
using TileSmall = Tile<64, 64, 32, 32>;    // decode-sized M
using TileLargeRow = Tile<128, 128, 64, 64, true>;
using TileSmallRow = Tile<64, 64, 32, 32, true>;

struct GemmArgs {
  const uint8_t* xq;
  const float* sa;
  const uint8_t* wq;
  const float* sw;
  int M, N, K, KB;
  void* y;
  int64_t ldy;
  int out_f32;
  float* ws;      // split-K partials (layout per kernel), or null
  int* counters;  // arrival counters of the decode path's output tiles, zero between calls
  int splits, kb_per_split;
  // grouped form
  const int32_t* offsets;
  int E;
  int64_t wq_stride, sw_stride;  // per expert
  int tiles_n;
  // grouped form with a row gather (or null): grouped row r reads the activation codes and
  // scales of source row rows[r], clamped to [0, src_rows - 1]
  const int32_t* rows;
  int src_rows;
  // decode GEMM with the activation quantization fused in: bf16 X rows (pitch ld_x) replace
  // xq / sa, and pow2 selects the scale format of its 1x128 groups
  const uint16_t* x;
  int64_t ld_x;
  int pow2;
};

template <class T>
struct Prefetch {
  uint4 a[T::A_LOADS];
  uint4 b[T::B_LOADS];
  float s;
  float sb;  // row-scaled B only
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <class T>
__device__ __forceinline__ void load_slice(Prefetch<T>& st, const uint8_t* A, int m_valid,
                                           const uint8_t* B, int n_valid, int64_t ld, const float* SA,
                                           const float* SB, int KB, int kb, int tid) {
  const int64_t koff = (int64_t)kb * 128;
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    const int c = tid + i * T::NT, row = c >> 3, cc = c & 7;
    st.a[i] = row < m_valid ? ldg16(A + row * ld + koff + cc * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < T::B_LOADS; ++i) {
    const int c = tid + i * T::NT, row = c >> 3, cc = c & 7;
    st.b[i] = row < n_valid ? ldg16(B + row * ld + koff + cc * 16) : make_uint4(0, 0, 0, 0);
  }
  st.s = (tid < T::BM && tid < m_valid) ? SA[(int64_t)tid * KB + kb] : 0.f;
  if constexpr (T::ROWB) st.sb = (tid < T::BN && tid < n_valid) ? SB[(int64_t)tid * KB + kb] : 0.f;
}

template <class T>
__device__ __forceinline__ void store_slice(const Prefetch<T>& st, uint8_t* stage, int tid) {
  uint8_t* sA = stage;
  uint8_t* sB = stage + T::A_BYTES;
  float* sS = reinterpret_cast<float*>(stage + T::A_BYTES + T::B_BYTES);
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    const int c = tid + i * T::NT, row = c >> 3, cc = c & 7;
    *reinterpret_cast<uint4*>(sA + row * 128 + ((cc ^ swz(row)) << 4)) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < T::B_LOADS; ++i) {
    const int c = tid + i * T::NT, row = c >> 3, cc = c & 7;
    *reinterpret_cast<uint4*>(sB + row * 128 + ((cc ^ swz(row)) << 4)) = st.b[i];
  }
  if (tid < T::BM) sS[tid] = st.s;
  if constexpr (T::ROWB)
    if (tid < T::BN) sS[T::BM + tid] = st.sb;
}

// Fragment of a 16x128 operand tile for v_mfma_f32_16x16x128_f8f6f4: lane l holds row l % 16 and
// the 32 consecutive k of quarter l / 16. A and B use the same k assignment, so the product sums
// every k of the slice exactly once.
__device__ __forceinline__ v8i load_frag(const uint8_t* s, int row, int kq) {
  const uint8_t* p = s + row * 128;
  const int sw = swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(p + (((2 * kq) ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(p + (((2 * kq + 1) ^ sw) << 4));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Exact widening of the four E4M3 codes in a dword to four f16 values (two per result).
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8h widen8_f16(int lo, int hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  v8h r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Sum over one 128-wide K slice for a 16x16 output tile.
//
// Fast form (PRECISE = false): one v_mfma_f32_16x16x128_f8f6f4. Its adder aligns the slice's
// products to the largest one and keeps about 15 bits below it (measured on gfx950), like the
// narrow FP8 accumulators the pages describe for other hardware; the per-slice promotion to the
// float32 accumulator bounds that loss to one slice.
//
// Precise form (PRECISE = true): the same codes widened exactly to f16 and summed by four
// v_mfma_f32_16x16x32_f16 (lane l's bytes 8s .. 8s+7 in step s, the same k for A and B), whose
// adder keeps float32-level precision.
template <bool PRECISE>
__device__ __forceinline__ v4f slice_product(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!PRECISE) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
  } else {
    v4f p = zero;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      p = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen8_f16(a[2 * s], a[2 * s + 1]),
                                                  widen8_f16(b[2 * s], b[2 * s + 1]), p, 0, 0, 0);
    return p;
  }
}

template <class T, bool PRECISE>
__device__ __forceinline__ void mma_slice(const uint8_t* stage, float swv, int wm, int wn, int lane,
                                          v4f (&acc)[T::TM][T::TN]) {
  const uint8_t* sA = stage;
  const uint8_t* sB = stage + T::A_BYTES;
  const float* sS = reinterpret_cast<const float*>(stage + T::A_BYTES + T::B_BYTES);
  const int r16 = lane & 15, kq = lane >> 4;
  v8i af[T::TM], bf[T::TN];
  v4f sc[T::TM];
  float sb[T::TN];  // row-scaled B: the scale of this lane's output column in sub-tile j
#pragma unroll
  for (int i = 0; i < T::TM; ++i) af[i] = load_frag(sA, wm * T::WM + i * 16 + r16, kq);
#pragma unroll
  for (int j = 0; j < T::TN; ++j) {
    bf[j] = load_frag(sB, wn * T::WN + j * 16 + r16, kq);
    sb[j] = T::ROWB ? sS[T::BM + wn * T::WN + j * 16 + r16] : 1.f;
  }
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
    // output rows of this lane in sub-tile i: 4 * kq + v, v = 0..3
    sc[i] = *reinterpret_cast<const v4f*>(sS + wm * T::WM + i * 16 + 4 * kq) * swv;
  }
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const v4f p = slice_product<PRECISE>(af[i], bf[j]);
      if constexpr (T::ROWB)
        acc[i][j] += p * (sc[i] * sb[j]);
      else
        acc[i][j] += p * sc[i];
    }
  }
}

// One output tile over K slices [kb0, kb1). A/SA start at the tile's first row, B at its first
// column (weight row); SW is the weight-scale matrix [N/128][KB] of the current expert, or, with
// row-scaled B, the tile's first row of sb [N][KB].
template <class T, bool PRECISE>
__device__ __forceinline__ void run_tile(const uint8_t* A, const float* SA, int m_valid,
                                         const uint8_t* B, const float* SW, int n0, int n_valid,
                                         int64_t ld, int KB, int kb0, int kb1, uint8_t* smem,
                                         v4f (&acc)[T::TM][T::TN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const float* swrow = T::ROWB ? nullptr : SW + (int64_t)((n0 + wn * T::WN) >> 7) * KB;

#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  if (kb0 >= kb1) return;

  Prefetch<T> st;
  load_slice<T>(st, A, m_valid, B, n_valid, ld, SA, SW, KB, kb0, tid);
  store_slice<T>(st, smem, tid);
  __syncthreads();
  for (int kb = kb0; kb < kb1; ++kb) {
    const int cur = (kb - kb0) & 1;
    const bool more = kb + 1 < kb1;
    if (more) load_slice<T>(st, A, m_valid, B, n_valid, ld, SA, SW, KB, kb + 1, tid);
    const float swv = T::ROWB ? 1.f : swrow[kb];
    mma_slice<T, PRECISE>(smem + cur * T::STAGE_BYTES, swv, wm, wn, lane, acc);
    if (more) store_slice<T>(st, smem + (cur ^ 1) * T::STAGE_BYTES, tid);
    __syncthreads();
  }
}

// Write a finished tile: rows [m0, m0 + m_valid) of Y (or of split-K partial `split`).
template <class T>
__device__ __forceinline__ void store_tile(const GemmArgs& p, int64_t row0, int m_valid, int n0,
                                           int split, const v4f (&acc)[T::TM][T::TN]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int r16 = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int col = n0 + wn * T::WN + j * 16 + r16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * T::WM + i * 16 + 4 * kq + v;
        if (r >= m_valid) continue;
        const int64_t row = row0 + r;
        const float val = acc[i][j][v];
        if (p.ws) {
          p.ws[((int64_t)split * p.M + row) * p.N + col] = val;
        } else if (p.out_f32) {
          reinterpret_cast<float*>(p.y)[row * p.ldy + col] = val;
        } else {
          reinterpret_cast<uint16_t*>(p.y)[row * p.ldy + col] = f32_to_bf16_rne(val);
        }
      }
    }
  }
}

// Map a linear workgroup id to (tile_m, tile_n). Ids are first regrouped so that each of the
// 8 XCDs (which receive workgroups round-robin) owns a contiguous range, then tiles are ordered in
// column groups of 8 m-tiles so that concurrently running workgroups on one XCD share A rows and
// B columns in that XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int total, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  constexpr int G = 8;
  const int per_group = G * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * G;
  const int gsize = min(tiles_m - first_m, G);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <class T, bool PRECISE>
__global__ __launch_bounds__(T::NT) void gemm_kernel(GemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tiles_m = (p.M + T::BM - 1) / T::BM;
  const int tiles_n = p.N / T::BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int split = blockIdx.y;
  const int kb0 = split * p.kb_per_split;
  const int kb1 = min(p.KB, kb0 + p.kb_per_split);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int m_valid = min(T::BM, p.M - m0);
  v4f acc[T::TM][T::TN];
  run_tile<T, PRECISE>(p.xq + (int64_t)m0 * p.K, p.sa + (int64_t)m0 * p.KB, m_valid,
              p.wq + (int64_t)n0 * p.K, T::ROWB ? p.sw + (int64_t)n0 * p.KB : p.sw, n0, T::BN,
              p.K, p.KB, kb0, kb1, smem, acc);
  store_tile<T>(p, m0, m_valid, n0, split, acc);
}

// ---------------------------------------------------------------------------------------------
// Large-M GEMM. Workgroup tiles of BM x BN (256 x 256 or 256 x 128) split over waves of
// WM x WN (128 x 64: 8 MFMA row tiles by 4 column tiles), so every LDS byte a wave reads feeds
// 1.5x (vs 64 x 64) more matrix-core work. K slices reach LDS by direct global->LDS DMA
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's base + 16 * lane), so
// staging costs no registers; the 16-byte chunk order inside each 128-byte row is the same XOR
// swizzle as above, applied on the global side. Two LDS stages as two separate arrays, with the
// K loop unrolled by two so that the stage each instruction touches is known statically (the
// compiler then does not have to wait for the in-flight DMA into the other stage before reading
// this one). Per K slice: wait for this wave's DMA, one barrier, start the next slice's DMA into
// the other stage, then multiply out of this stage.
// ---------------------------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, bool ROWB_ = false>
struct Big {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr bool ROWB = ROWB_;  // B scales per row and slice (see Tile)
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int NT = WAVES * 64;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, S_BYTES = BM * 4;
  static constexpr int SB_BYTES = ROWB ? BN * 4 : 0;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES + SB_BYTES;
  static constexpr int A_PER_WAVE = BM / 8 / WAVES;  // one DMA instruction moves 8 rows (1 KiB)
  static constexpr int B_PER_WAVE = BN / 8 / WAVES;
  static constexpr int S_ROWS = BM / WAVES;  // activation scales loaded per wave
  static constexpr int SB_ROWS = BN / WAVES;  // row-scaled B: B scales loaded per wave
  static constexpr int DMA_OPS = A_PER_WAVE + B_PER_WAVE + 1 + (ROWB ? 1 : 0);  // per wave, slice
  static_assert(STAGES >= 2 && STAGES <= 3, "waits are written out for up to one slice ahead");
  static_assert(A_PER_WAVE * 8 * WAVES == BM && B_PER_WAVE * 8 * WAVES == BN, "DMA split");
  static_assert(S_ROWS <= 64 && S_ROWS * WAVES == BM, "scale DMA split");
  static_assert(SB_ROWS <= 64 && SB_ROWS * WAVES == BN, "B-scale DMA split");
  static_assert(128 % WN == 0, "a wave's columns must share one weight-scale block");
};

constexpr int kMaxSlices = 256;  // K <= 32768 on the large-tile path
constexpr int kMaxExperts = 1024;
using BigWide = Big<256, 256, 128, 64, 2>;    // 8 waves
using BigNarrow = Big<256, 128, 128, 64, 2>;  // 4 waves
using BigGroup = Big<128, 256, 64, 64, 3>;    // 8 waves; grouped GEMM (expert segments are short)
using BigWideRow = Big<256, 256, 128, 64, 2, true>;
using BigNarrowRow = Big<256, 128, 128, 64, 2, true>;
// f16 slice sums: the widened fragments take twice the registers, so 8 waves of 64x64 and three
// stages (8-10 % faster than 4 waves of 128x64 with two stages on the 8192-row GEMMs)
using BigF16 = Big<256, 128, 64, 64, 3>;
using BigF16Row = Big<256, 128, 64, 64, 3, true>;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS DMA of 16 (or 4) bytes per lane from base + off (off a per-lane 32-bit byte
// offset, base wave-uniform): lane l's bytes land at lds + 16 * l (4 * l); `lds` must be the same
// for the whole wave (it goes to M0). Written as inline assembly so that the compiler does not
// track these loads: it would otherwise wait for every DMA in flight before any later LDS read,
// even of the other stage. Completion is waited for explicitly (wait_dma_and_barrier) before the
// stage is read.
__device__ __forceinline__ uint32_t lds_offset(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}
// The base address is wave-uniform; readfirstlane states that to the compiler, which must hold
// it in scalar registers for the instruction's saddr operand.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// The LDS address goes to M0 through an explicit register constraint, so the compiler sets M0
// itself and knows it is read here. The compiler cannot see the instruction inside the asm, so it
// inserts none of the wait states the hardware needs before it: the base address SGPRs are often
// written by v_readfirstlane right before (a VALU write of an SGPR that a vector-memory
// instruction reads needs 5 wait states; without them the DMA can take a stale base address and
// fault), and M0 by an SALU instruction (1 wait state). s_nop 4 provides the 5 in every case.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, const uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "{m0}"(m0v) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, const uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(uniform_ptr(base)), "{m0}"(m0v) : "memory");
}

// Per-lane byte offsets of this lane's DMA sources within a K slice (computed once per tile).
// Rows past the end of the matrix are clamped to its last row: they load valid memory whose
// products only reach output rows / columns that are never stored. With a row gather (g
// non-null: the source rows of this lane's A and scale DMA, as loaded from the gather list) the
// A and scale offsets are those of the source rows, relative to the start of the source matrix.
template <class T>
struct GatherRows {
  int a[T::A_PER_WAVE];
  int s;
};

template <class T>
struct DmaPlan {
  uint32_t a[T::A_PER_WAVE];
  uint32_t b[T::B_PER_WAVE];
  uint32_t s;
  uint32_t sb;  // row-scaled B
};

// The entries of a tile's gather list (rows: the tile's first entry) that this lane's A and
// scale DMA read, as loaded (clamped when the plan is made).
template <class T>
__device__ __forceinline__ GatherRows<T> load_gather_rows(const int32_t* rows, int m_valid,
                                                          int wave, int lane) {
  GatherRows<T> g;
#pragma unroll
  for (int t = 0; t < T::A_PER_WAVE; ++t)
    g.a[t] = rows[min((t * T::WAVES + wave) * 8 + (lane >> 3), m_valid - 1)];
  g.s = rows[min(wave * T::S_ROWS + lane, m_valid - 1)];
  return g;
}

template <class T>
__device__ __forceinline__ DmaPlan<T> make_dma_plan(int m_valid, int n_valid, int K, int KB,
                                                    int wave, int lane,
                                                    const GatherRows<T>* g = nullptr,
                                                    int src_rows = 0) {
  DmaPlan<T> d;
  const int sub = lane >> 3;
  // source row of tile row trow (gather entry v), clamped to the matrix (the caller bounds
  // src_rows * K and src_rows * KB * 4 below 2^32)
  auto src = [&](int trow, int v) -> uint32_t {
    return g ? (uint32_t)min(max(v, 0), src_rows - 1) : (uint32_t)min(trow, m_valid - 1);
  };
  // lane l fills LDS slot l & 7 of tile row 8 * ins + (l >> 3): it loads the logical chunk that
  // the swizzle puts there (the row used for the swizzle is the unclamped tile row)
#pragma unroll
  for (int t = 0; t < T::A_PER_WAVE; ++t) {
    const int trow = (t * T::WAVES + wave) * 8 + sub;
    const int cc = (lane & 7) ^ swz(trow);
    d.a[t] = src(trow, g ? g->a[t] : 0) * (uint32_t)K + (uint32_t)(cc * 16);
  }
#pragma unroll
  for (int t = 0; t < T::B_PER_WAVE; ++t) {
    const int trow = (t * T::WAVES + wave) * 8 + sub;
    const int cc = (lane & 7) ^ swz(trow);
    d.b[t] = (uint32_t)(min(trow, n_valid - 1) * K + cc * 16);
  }
  d.s = src(wave * T::S_ROWS + lane, g ? g->s : 0) * (uint32_t)(KB * 4);
  d.sb = (uint32_t)(min(wave * T::SB_ROWS + lane, n_valid - 1) * KB * 4);
  return d;
}

template <class T>
__device__ __forceinline__ void dma_slice(uint8_t* stage, const DmaPlan<T>& d, const uint8_t* A,
                                          const uint8_t* B, const float* SA, const float* SB,
                                          int kb, int wave, int lane) {
  const uint8_t* a = A + (int64_t)kb * 128;
  const uint8_t* b = B + (int64_t)kb * 128;
  // the scale DMA goes first: anything the compiler has to wait for before computing its
  // operands (e.g. a reloaded register) then does not wait on this slice's tile DMA as well
  if (lane < T::S_ROWS)
    dma4(SA + kb, d.s, stage + T::A_BYTES + T::B_BYTES + wave * T::S_ROWS * 4);
  if constexpr (T::ROWB)
    if (lane < T::SB_ROWS)
      dma4(SB + kb, d.sb, stage + T::A_BYTES + T::B_BYTES + T::S_BYTES + wave * T::SB_ROWS * 4);
#pragma unroll
  for (int t = 0; t < T::A_PER_WAVE; ++t) dma16(a, d.a[t], stage + (t * T::WAVES + wave) * 1024);
#pragma unroll
  for (int t = 0; t < T::B_PER_WAVE; ++t)
    dma16(b, d.b[t], stage + T::A_BYTES + (t * T::WAVES + wave) * 1024);
}

// Wait for this wave's outstanding DMA and LDS operations, then a workgroup barrier. The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_dma_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The same, but leaving the DMAs of the next `ahead` slices (issued after the awaited one) in
// flight: vector-memory operations complete in order, so at most that many may be outstanding.
template <class T>
__device__ __forceinline__ void wait_slice_and_barrier(int ahead) {
  if (T::STAGES >= 3 && ahead >= 1)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(T::DMA_OPS) : "memory");
  else
    wait_dma_and_barrier();
}

// One K slice of a wave's WM x WN tile, software-pipelined by row tile: the matrix-core sums of
// row tile i are issued interleaved with the scale-and-accumulate FMAs of row tile i - 1 (whose
// sums finished long before), so the VALU works while the matrix core runs and no FMA waits on
// the sum it consumes; the next row tile's operands are read from LDS meanwhile. Scheduling
// fences keep the compiler from regrouping the FMAs next to the sums they depend on.
template <class T, int ACC>
__device__ __forceinline__ void mma_slice_big(const uint8_t* stage, float swv, int wm, int wn,
                                              int lane, v4f (&acc)[T::TM][T::TN]) {
  constexpr bool PRECISE = ACC == 1;
  const uint8_t* sA = stage;
  const uint8_t* sB = stage + T::A_BYTES;
  const float* sS = reinterpret_cast<const float*>(stage + T::A_BYTES + T::B_BYTES);
  const float* sSB = sS + T::BM;  // row-scaled B: this slice's scales of the tile's B rows
  const int r16 = lane & 15, kq = lane >> 4;
  v8i bf[T::TN];
  float sb[T::TN];  // row-scaled B: the scale of this lane's output column in sub-tile j
#pragma unroll
  for (int j = 0; j < T::TN; ++j) {
    bf[j] = load_frag(sB, wn * T::WN + j * 16 + r16, kq);
    sb[j] = T::ROWB ? sSB[wn * T::WN + j * 16 + r16] : 1.f;
  }
  if constexpr (ACC == 2) {
    // power-of-two scales: lane l's E8M0 exponents scale A row l % 16 and B column l % 16 of
    // every 32-wide K block it holds; the instruction adds the running sum itself
    int sbe[T::TN];  // B exponent of this lane's column: one per block, or one per row
#pragma unroll
    for (int j = 0; j < T::TN; ++j) sbe[j] = e8m0_of(T::ROWB ? sb[j] : swv);
    int sae[T::TM];  // every row tile's scale exponent, read with the B fragments
#pragma unroll
    for (int i = 0; i < T::TM; ++i) sae[i] = e8m0_of(sS[wm * T::WM + i * 16 + r16]);
    // row tile i + 1's fragment is read while row tile i's products run (separate registers)
    v8i af = load_frag(sA, wm * T::WM + r16, kq);
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
      v8i af_next = af;
      if (i + 1 < T::TM) af_next = load_frag(sA, wm * T::WM + (i + 1) * 16 + r16, kq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0,
                                                                     sae[i], 0, sbe[j]);
      __builtin_amdgcn_sched_barrier(0);
      af = af_next;
    }
    return;
  }
  v8i af = load_frag(sA, wm * T::WM + r16, kq);
  v4f sc = *reinterpret_cast<const v4f*>(sS + wm * T::WM + 4 * kq) * swv;
  v4f p_prev[T::TN];
  v4f sc_prev = sc;
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
    v8i af_next = af;
    v4f sn = sc;
    if (i + 1 < T::TM) {
      af_next = load_frag(sA, wm * T::WM + (i + 1) * 16 + r16, kq);
      sn = *reinterpret_cast<const v4f*>(sS + wm * T::WM + (i + 1) * 16 + 4 * kq);
    }
    v4f p_cur[T::TN];
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      p_cur[j] = slice_product<PRECISE>(af, bf[j]);
      __builtin_amdgcn_sched_barrier(0);
      if (i > 0) {
        if constexpr (T::ROWB)
          acc[i - 1][j] += p_prev[j] * (sc_prev * sb[j]);
        else
          acc[i - 1][j] += p_prev[j] * sc_prev;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < T::TN; ++j) p_prev[j] = p_cur[j];
    sc_prev = sc;
    af = af_next;
    sc = sn * swv;
  }
#pragma unroll
  for (int j = 0; j < T::TN; ++j) {
    if constexpr (T::ROWB)
      acc[T::TM - 1][j] += p_prev[j] * (sc_prev * sb[j]);
    else
      acc[T::TM - 1][j] += p_prev[j] * sc_prev;
  }
}

// Row pitch (bf16 elements) of the output tile staged in LDS by the bf16 epilogue: 8 bytes of
// padding per row spread the column-wise writes over the banks and keep rows 8-byte aligned.
template <class T>
constexpr int kEpiPitch = T::BN + 4;

// One BM x BN output tile over all K slices: operands DMA'd through STAGES LDS stages (the next
// STAGES - 1 slices in flight while slice kb is multiplied), the weight scales of the tile's (up to two)
// 128-column blocks read into LDS once. A / SA start at the tile's first row, B at its first
// column (weight row); SW is the weight-scale matrix [N/128][KB] (of the tile's expert); Y rows
// y_row0 + r, r < m_valid, pitch ldy. The caller's previous use of the LDS arrays must be over.
// Weight scales of the tile's (up to two) 128-column blocks into LDS, and the tile's DMA plan.
template <class T>
__device__ __forceinline__ DmaPlan<T> big_tile_prepare(const GemmArgs& p,
                                                       float (*sw_s)[kMaxSlices], const float* SW,
                                                       int n0, int m_valid, int n_valid) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = p.KB;
  // a wave whose columns are all past N still runs (it takes part in the DMA and barriers) on a
  // clamped scale row; its results are not stored
  constexpr int NBLK = (T::BN + 127) / 128;
  if constexpr (!T::ROWB) {
    for (int e = tid; e < NBLK * KB; e += T::NT) {
      const int b = e / KB, k = e - (e / KB) * KB;
      const int nb = min((n0 >> 7) + b, p.N / 128 - 1);
      sw_s[b][k] = SW[(int64_t)nb * KB + k];
    }
  }
  return make_dma_plan<T>(m_valid, n_valid, p.K, KB, wave, lane);
}

// The tile's multiply-accumulate and store. dma0_done: slice 0 is already on its way into stage
// 0 (issued by the caller). on_loop_end runs once every wave is past the last slice -- the
// stages are free then -- and before the epilogue, which stages the bf16 tile in LDS from byte
// epi_off (so a caller may start the next tile's slice 0 into stage 0 meanwhile).
template <class T, int ACC, class OnLoopEnd>
__device__ __forceinline__ void big_tile_core(const GemmArgs& p, uint8_t* stages,
                                              float (*sw_s)[kMaxSlices], const DmaPlan<T>& dp,
                                              const uint8_t* A, const float* SA, int m_valid,
                                              const uint8_t* B, const float* SW, int n0,
                                              int n_valid, int64_t y_row0, bool dma0_done,
                                              int epi_off, OnLoopEnd on_loop_end) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int KB = p.KB;
  const float* swrow = sw_s[((n0 + wn * T::WN) >> 7) - (n0 >> 7)];
  // row-scaled B: the tile's rows of sb [N][KB] travel with each slice instead
  const float* SB = T::ROWB ? SW + (int64_t)n0 * KB : nullptr;

  v4f acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  if constexpr (T::STAGES == 2) {
    uint8_t* const stage0 = stages;
    uint8_t* const stage1 = stages + T::STAGE_BYTES;
    if (!dma0_done) dma_slice<T>(stage0, dp, A, B, SA, SB, 0, wave, lane);
    for (int kb = 0; kb < KB; kb += 2) {
      wait_dma_and_barrier();
      if (kb + 1 < KB) dma_slice<T>(stage1, dp, A, B, SA, SB, kb + 1, wave, lane);
      mma_slice_big<T, ACC>(stage0, T::ROWB ? 1.f : swrow[kb], wm, wn, lane, acc);
      if (kb + 1 >= KB) break;
      wait_dma_and_barrier();
      if (kb + 2 < KB) dma_slice<T>(stage0, dp, A, B, SA, SB, kb + 2, wave, lane);
      mma_slice_big<T, ACC>(stage1, T::ROWB ? 1.f : swrow[kb + 1], wm, wn, lane, acc);
    }
  } else {
    // slices kb + 1 and kb + 2 in flight while kb is multiplied
    if (!dma0_done) dma_slice<T>(stages, dp, A, B, SA, SB, 0, wave, lane);
    if (KB > 1) dma_slice<T>(stages + T::STAGE_BYTES, dp, A, B, SA, SB, 1, wave, lane);
    int cur = 0;
    for (int kb = 0; kb < KB; ++kb) {
      wait_slice_and_barrier<T>(KB - 1 - kb);
      const int nxt = cur == 0 ? 2 : cur - 1;  // (kb + 2) % 3
      if (kb + 2 < KB) dma_slice<T>(stages + nxt * T::STAGE_BYTES, dp, A, B, SA, SB, kb + 2, wave, lane);
      mma_slice_big<T, ACC>(stages + cur * T::STAGE_BYTES, T::ROWB ? 1.f : swrow[kb], wm, wn, lane, acc);
      cur = cur == 2 ? 0 : cur + 1;
    }
  }

  const int r16 = lane & 15, kq = lane >> 4;
  if (!p.out_f32) {
    // bf16 output: the tile is rounded into LDS (the stages are free once every wave is past its
    // last slice), then leaves as whole 16-byte pieces of rows instead of 2-byte stores
    uint16_t* t16 = reinterpret_cast<uint16_t*>(stages + epi_off);
    __syncthreads();
    on_loop_end();
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          t16[(wm * T::WM + i * 16 + 4 * kq + v) * kEpiPitch<T> + wn * T::WN + j * 16 + r16] =
              f32_to_bf16_rne(acc[i][j][v]);
    __syncthreads();
    constexpr int CH = T::BN / 8;  // 16-byte pieces per row
    for (int q = tid; q < T::BM * CH; q += T::NT) {
      const int r = q / CH, c8 = (q - (q / CH) * CH) * 8;
      if (r >= m_valid || c8 >= n_valid) continue;
      const uint16_t* src = t16 + r * kEpiPitch<T> + c8;  // 8-byte aligned
      const u32x2 lo = *reinterpret_cast<const u32x2*>(src);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 4);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.y) + (y_row0 + r) * p.ldy + n0 + c8) =
          u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    return;
  }
  __syncthreads();
  on_loop_end();
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int c = wn * T::WN + j * 16 + r16;
      if (c >= n_valid) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = wm * T::WM + i * 16 + 4 * kq + v;
        if (r >= m_valid) continue;
        reinterpret_cast<float*>(p.y)[(y_row0 + r) * p.ldy + n0 + c] = acc[i][j][v];
      }
    }
  }
}

template <class T, int ACC>
__global__ __launch_bounds__(T::NT) void gemm_big_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t stages[T::STAGES * T::STAGE_BYTES];
  __shared__ float sw_s[(T::BN + 127) / 128][kMaxSlices];
  const int tiles_m = (p.M + T::BM - 1) / T::BM;
  const int tiles_n = (p.N + T::BN - 1) / T::BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int m_valid = min(T::BM, p.M - m0), n_valid = min(T::BN, p.N - n0);
  static_assert(T::BM * kEpiPitch<T> * 2 <= T::STAGES * T::STAGE_BYTES, "epilogue tile fits");
  const DmaPlan<T> dp = big_tile_prepare<T>(p, sw_s, p.sw, n0, m_valid, n_valid);
  big_tile_core<T, ACC>(p, stages, sw_s, dp, p.xq + (int64_t)m0 * p.K, p.sa + (int64_t)m0 * p.KB,
                        m_valid, p.wq + (int64_t)n0 * p.K, p.sw, n0, n_valid, m0, false, 0,
                        [] {});
}

// Grouped GEMM on the DMA-fed tiles, persistent: a fixed grid of workgroups walks the list of
// (expert m-tile, n-tile) pairs. Each workgroup first forms, from the device offsets, the
// clamped offsets and the prefix sums of the per-expert m-tile counts in LDS (once), then finds
// each tile's expert by binary search there. The tile list is cut into one contiguous chunk per
// XCD (workgroup w runs on XCD w % 8), so the m-tiles of one expert -- which read the same weight
// panels -- and the n-tiles of one m-tile -- which read the same activation rows -- share an L2.
// The global values a tile's set-up needs (its weight-block scales and, with a row gather, its
// source rows) are loaded when the tile before it starts, so that the next tile's first slice
// DMA goes out at the end of the current tile's K loop without a memory round trip.
template <class T, int ACC>
__global__ __launch_bounds__(T::NT) void grouped_big_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t stages[T::STAGES * T::STAGE_BYTES];
  __shared__ float sw_s[(T::BN + 127) / 128][kMaxSlices];
  __shared__ int s_first[kMaxExperts + 1];  // m-tiles of experts before e
  __shared__ int s_lo[kMaxExperts + 1];     // first row of expert e (offsets clamped to [0, M])
  int* const s_part = reinterpret_cast<int*>(stages);  // scan scratch (before any DMA)
  static_assert(T::NT * sizeof(int) <= T::STAGES * T::STAGE_BYTES, "scan scratch fits");
  const int tid = threadIdx.x;
  const int E = p.E;
  // prefix sums of ceil(rows_e / BM), NT experts per pass (E <= kMaxExperts); expert e's rows
  // are [s_lo[e], max(s_lo[e + 1], s_lo[e]))
  int carry = 0;
  for (int base = 0; base < E; base += T::NT) {
    const int e = base + tid;
    int cnt = 0;
    if (e < E) {
      const int lo = min(max(p.offsets[e], 0), p.M);
      const int hi = min(max(p.offsets[e + 1], lo), p.M);
      cnt = (hi - lo + T::BM - 1) / T::BM;
      s_lo[e] = lo;
    }
    s_part[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < T::NT; d <<= 1) {
      const int v = tid >= d ? s_part[tid - d] : 0;
      __syncthreads();
      s_part[tid] += v;
      __syncthreads();
    }
    if (e < E) s_first[e] = carry + s_part[tid] - cnt;
    carry += s_part[T::NT - 1];
    __syncthreads();
  }
  if (tid == 0) {
    s_first[E] = carry;
    s_lo[E] = min(max(p.offsets[E], 0), p.M);
  }
  __syncthreads();
  const int tiles_n = p.tiles_n;
  const int total = s_first[E] * tiles_n;
  const int G = gridDim.x, per_xcd = G / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int chunk = (total + 7) / 8;
  const int t_end = min(total, (xcd + 1) * chunk);
  // tile t -> (expert e, first row, valid rows, first column), from LDS only
  struct Coords {
    int e, row0, m_valid, n0, n_valid;
  };
  auto coords = [&](int t) {
    const int tm_lin = t / tiles_n, tn = t - (t / tiles_n) * tiles_n;
    // expert e: s_first[e] <= tm_lin < s_first[e + 1]
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_first[mid] <= tm_lin) lo = mid; else hi = mid;
    }
    // every lane computes the same values; readfirstlane tells the compiler so (the DMA bases
    // must be scalar registers)
    Coords c;
    c.e = __builtin_amdgcn_readfirstlane(lo);
    const int r_lo = s_lo[c.e];
    const int r_hi = max(s_lo[c.e + 1], r_lo);
    c.row0 = __builtin_amdgcn_readfirstlane(r_lo + (tm_lin - s_first[c.e]) * T::BM);
    c.m_valid = __builtin_amdgcn_readfirstlane(min(T::BM, r_hi - c.row0));
    c.n0 = __builtin_amdgcn_readfirstlane(tn * T::BN);
    c.n_valid = __builtin_amdgcn_readfirstlane(min(T::BN, p.N - c.n0));
    return c;
  };
  const uint8_t* const wq0 = p.wq;
  // with a row gather the DMA offsets address the source rows from the start of xq / sa
  const bool gather = p.rows != nullptr;
  auto a_of = [&](const Coords& c) { return gather ? p.xq : p.xq + (int64_t)c.row0 * p.K; };
  auto sa_of = [&](const Coords& c) { return gather ? p.sa : p.sa + (int64_t)c.row0 * p.KB; };
  auto b_of = [&](const Coords& c) { return wq0 + c.e * p.wq_stride + (int64_t)c.n0 * p.K; };
  auto sw_of = [&](const Coords& c) { return p.sw + c.e * p.sw_stride; };
  // A tile's set-up in two halves. fetch: the global loads (thread tid < NBLK KB loads weight-
  // block scale tid -- NBLK <= 2 column blocks x KB <= 256 slices <= NT values -- and the other
  // threads a copy of the last one; with a row gather, every lane its rows' gather entries).
  // commit: the scales into LDS (the previous tile's K loop is done with them) and the DMA plan.
  constexpr int NBLK = (T::BN + 127) / 128;
  static_assert(NBLK * kMaxSlices <= T::NT, "one weight-block scale per thread");
  static_assert(!T::ROWB, "grouped GEMM: block-scaled weights");
  const int KB = p.KB;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  struct Fetch {
    float sw;
    GatherRows<T> g;
  };
  auto fetch = [&](const Coords& c) {
    Fetch f;
    {  // every thread loads (threads past NBLK KB a repeat): no register write precedes the load
      const int e = min(tid, NBLK * KB - 1);
      const int b = e / KB, k = e - (e / KB) * KB;
      const int nb = min((c.n0 >> 7) + b, p.N / 128 - 1);
      f.sw = sw_of(c)[(int64_t)nb * KB + k];
    }
    if (gather) f.g = load_gather_rows<T>(p.rows + c.row0, c.m_valid, wave, lane);
    return f;
  };
  auto commit = [&](const Coords& c, Fetch f) {
    // the fetched values are taken here, on every path: the empty asm statements keep the
    // compiler from moving any use of them -- and with it the wait for their loads, which would
    // also wait for the slice DMA in flight -- to the top of the tile
    asm volatile("" : "+v"(f.sw));
    if (gather) {
#pragma unroll
      for (int i = 0; i < T::A_PER_WAVE; ++i) asm volatile("" : "+v"(f.g.a[i]));
      asm volatile("" : "+v"(f.g.s));
    }
    if (tid < NBLK * KB) sw_s[tid / KB][tid - (tid / KB) * KB] = f.sw;
    return make_dma_plan<T>(c.m_valid, c.n_valid, p.K, KB, wave, lane, gather ? &f.g : nullptr,
                            p.src_rows);
  };
  // The next tile's slice 0 goes out into stage 0 while this tile's epilogue works in the
  // stages behind it (when the staged tile fits there): each tile's DMA start-up hides behind
  // the previous tile's store phase.
  constexpr bool kAhead = T::STAGE_BYTES + T::BM * kEpiPitch<T> * 2 <= T::STAGES * T::STAGE_BYTES;
  static_assert(T::BM * kEpiPitch<T> * 2 <= T::STAGES * T::STAGE_BYTES, "epilogue tile fits");
  int t = xcd * chunk + slot;
  if (t >= t_end) return;
  Coords c = coords(t);
  DmaPlan<T> dp = commit(c, fetch(c));
  if (kAhead) dma_slice<T>(stages, dp, a_of(c), b_of(c), sa_of(c), nullptr, 0, wave, lane);
  for (;;) {
    const int t_next = t + per_xcd;
    const bool more = t_next < t_end;
    // fetched and committed on every path (the last tile re-fetches its own values), so that
    // no load is left pending across the loop's back edge: the compiler would otherwise wait
    // for all memory operations, the slice DMA in flight included, at the top of each tile
    const Coords cn = coords(more ? t_next : t);
    const Fetch fn = fetch(cn);
    DmaPlan<T> dpn = dp;
    big_tile_core<T, ACC>(p, stages, sw_s, dp, a_of(c), sa_of(c), c.m_valid, b_of(c), sw_of(c),
                          c.n0, c.n_valid, c.row0, kAhead, kAhead ? T::STAGE_BYTES : 0, [&] {
                            if (!kAhead) return;
                            dpn = commit(cn, fn);
                            if (more)
                              dma_slice<T>(stages, dpn, a_of(cn), b_of(cn), sa_of(cn), nullptr,
                                           0, wave, lane);
                          });
    if (!more) break;
    __syncthreads();  // the epilogue's LDS reads are done before the next tile's DMA lands there
    t = t_next;
    c = cn;
    dp = kAhead ? dpn : commit(c, fn);
  }
}

// A GEMM workspace starts with a header of arrival counters, one per output tile of the split-K
// decode GEMM (which therefore splits K only while it has at most kWsCounters tiles); partials
// follow.
constexpr size_t kWsHeaderBytes = 4096;
constexpr int64_t kWsCounters = kWsHeaderBytes / sizeof(int);

__device__ __forceinline__ v8i load_frag_global(const uint8_t* row_base, int kb, int kq) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row_base + (int64_t)kb * 128 + kq * 32);
  const u32x4 lo = __builtin_nontemporal_load(p), hi = __builtin_nontemporal_load(p + 1);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// ---------------------------------------------------------------------------------------------
// Decode-sized GEMM (5 <= M <= 64): weight streaming on DMA-fed tiles. Workgroup (t, s) computes
// the BM x BN output tile t (BM = M padded to 32 or 64 rows, BN = 64 or 128 columns) over K
// slices [s L, s L + L) with KH halves of 4 waves (BN / 4 columns per wave): each half streams
// its own part of the range through its own stages, and the halves' partial tiles are summed
// through LDS in half order. Both operands of a slice reach LDS as in the large-M GEMM (global_load_lds_dwordx4, so each load instruction reads whole 128-byte
// rows; fragment loads straight into registers, where a quarter-wave touches 16 rows, stream
// the weights more slowly), through three stages: two slices in flight while one is multiplied.
// Each wave's weight-block scale travels with the slice (one 4-byte DMA per wave), so the K
// loop issues no other memory access. Every weight byte is read from HBM once.
//
// K splits (S > 1): each split stores its float32 partial tile with agent-scope stores into
// slot (t, s) of the workspace and bumps the tile's arrival counter; the split that arrives
// last reads the partials back, sums them in split order -- the same bits whatever the arrival
// order -- writes Y and re-arms the counter for the next call.
// ---------------------------------------------------------------------------------------------
template <int BM_, int BN_, int WN_, int KH_ = 1>
struct Dec : Big<BM_, BN_, BM_, WN_, 3> {
  using Base = Big<BM_, BN_, BM_, WN_, 3>;
  // KH halves of 4 waves per workgroup, each streaming its own part of the K range through its
  // own stages; the halves' partial tiles are summed through LDS in half order
  static constexpr int KH = KH_;
  static constexpr int NT = Base::NT * KH;
  static constexpr int SW_OFF = Base::STAGE_BYTES;  // one weight-block scale per wave
  static constexpr int STAGE_BYTES = SW_OFF + 16 * ((Base::WAVES * 4 + 15) / 16);
  static constexpr int DMA_OPS = Base::DMA_OPS + 1;  // per wave and slice
  static constexpr int SLOT_FLOATS = BM_ * BN_;      // one partial tile
  static constexpr int NV = Base::TM * Base::TN * 4;  // accumulator values per lane
  static_assert(Base::WAVES_M == 1 && NV <= 32, "waves side by side along N");
};

template <class T, int ACC>
__global__ __launch_bounds__(T::NT) void gemm_decode_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::KH * T::STAGES * T::STAGE_BYTES];
  __shared__ int s_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int half = __builtin_amdgcn_readfirstlane(tid >> 8);  // 0 unless KH = 2
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // wave within the half
  uint8_t* const stages = lds + half * (T::STAGES * T::STAGE_BYTES);
  const int t = blockIdx.x, split = blockIdx.y;
  const int kbs = split * p.kb_per_split;
  const int nks = min(p.kb_per_split, p.KB - kbs);  // >= 1: the plan leaves no empty range
  // this half's slices: the first ceil(nks / KH) of the range, or the rest (possibly none);
  // both halves run the same number of trips so that they meet at every barrier
  const int trips = (nks + T::KH - 1) / T::KH;
  const int kb0 = kbs + half * trips;
  const int nk = half == 0 ? trips : nks - trips;
  const int n0 = t * T::BN;
  const DmaPlan<T> dp = make_dma_plan<T>(p.M, T::BN, p.K, p.KB, wave, lane);
  const uint8_t* B = p.wq + (int64_t)n0 * p.K;
  // byte offset of this wave's weight-block scale row in sw (its lane 0 loads the slice's scale)
  const uint32_t sw_off = (uint32_t)((n0 + wave * T::WN) >> 7) * (uint32_t)(p.KB * 4);
  auto dma = [&](uint8_t* stage, int kb) {
    dma_slice<T>(stage, dp, p.xq, B, p.sa, nullptr, kb, wave, lane);
    if (lane == 0) dma4(p.sw + kb, sw_off, stage + T::SW_OFF + wave * 4);
  };

  v4f acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  constexpr int P = T::STAGES - 1;  // slices issued ahead of the one multiplied
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (u < nk) dma(stages + u * T::STAGE_BYTES, kb0 + u);
  int cur = 0;
  for (int i = 0; i < trips; ++i) {
    wait_slice_and_barrier<T>(nk - 1 - i);  // slice i + 1 may stay in flight
    const int nxt = cur == 0 ? P : cur - 1;  // (i + P) % STAGES: freed by slice i - 1
    if (i + P < nk) dma(stages + nxt * T::STAGE_BYTES, kb0 + i + P);
    if (i < nk) {
      const uint8_t* st = stages + cur * T::STAGE_BYTES;
      const float swv = reinterpret_cast<const float*>(st + T::SW_OFF)[wave];
      mma_slice_big<T, ACC>(st, swv, 0, wave, lane, acc);
    }
    cur = cur == P ? 0 : cur + 1;
  }

  const int r16 = lane & 15, kq = lane >> 4;
  float vals[T::NV];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) vals[(i * T::TN + j) * 4 + v] = acc[i][j][v];
  if constexpr (T::KH == 2) {
    // half 1's partial tile through LDS (every wave is past its last slice), added to half 0's
    float* red = reinterpret_cast<float*>(lds) + (wave * T::NV) * 64 + lane;
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int q = 0; q < T::NV; ++q) red[q * 64] = vals[q];
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int q = 0; q < T::NV; ++q) vals[q] += red[q * 64];
    }
  }
  const bool owner = half == 0;  // holds the tile's values from here on
  // The output tile goes through LDS (the stages are free once every wave is past its last
  // slice) and leaves as 16-byte pieces of rows.
  static_assert(T::BM * (T::BN + 4) * 4 <= T::STAGES * T::STAGE_BYTES, "output tile fits");
  auto store_y = [&]() {
    __syncthreads();
    if (p.out_f32) {
      constexpr int PITCH = T::BN + 4;  // floats; rows stay 16-byte aligned
      float* t32 = reinterpret_cast<float*>(lds);
      if (owner)
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              t32[(i * 16 + 4 * kq + v) * PITCH + wave * T::WN + j * 16 + r16] =
                  vals[(i * T::TN + j) * 4 + v];
      __syncthreads();
      constexpr int CH = T::BN / 4;
      for (int q = tid; q < T::BM * CH; q += T::NT) {
        const int r = q / CH, c = (q - r * CH) * 4;
        if (r >= p.M) break;  // q grows with r
        *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(p.y) + r * p.ldy + n0 + c) =
            *reinterpret_cast<const u32x4*>(t32 + r * PITCH + c);
      }
    } else {
      constexpr int PITCH = T::BN + 8;  // bf16 elements; rows stay 16-byte aligned
      uint16_t* t16 = reinterpret_cast<uint16_t*>(lds);
      if (owner)
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              t16[(i * 16 + 4 * kq + v) * PITCH + wave * T::WN + j * 16 + r16] =
                  f32_to_bf16_rne(vals[(i * T::TN + j) * 4 + v]);
      __syncthreads();
      constexpr int CH = T::BN / 8;
      for (int q = tid; q < T::BM * CH; q += T::NT) {
        const int r = q / CH, c = (q - r * CH) * 8;
        if (r >= p.M) break;
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.y) + r * p.ldy + n0 + c) =
            *reinterpret_cast<const u32x4*>(t16 + r * PITCH + c);
      }
    }
  };
  const int S = gridDim.y;
  if (S == 1) {
    store_y();
    return;
  }
  // partial tile of (t, split): value q of lane l of wave w at float (w * NV + q) * 64 + l
  float* base = p.ws + (size_t)wave * T::NV * 64 + lane;
  float* mine = base + ((size_t)t * S + split) * T::SLOT_FLOATS;
  if (owner)
#pragma unroll
    for (int q = 0; q < T::NV; ++q)
      __hip_atomic_store(mine + q * 64, vals[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Ordering of the hand-off. Every access to the partials and the counter is an agent-scope
  // atomic: the partial stores are write-through stores (sc1) that complete only once they have
  // reached the level all XCDs share, and the read-back loads (sc1) are served from that level,
  // never from a stale L2 line. The s_waitcnt below completes this thread's partial stores
  // before the barrier, so every partial of this split is visible agent-wide before thread 0
  // issues the arrival RMW; the last arrival issues its loads only after that RMW has returned
  // (its result reaches the other threads through LDS and a barrier). The RMW is therefore
  // relaxed: release / acquire ordering at agent scope would add a writeback of the whole L2 and
  // invalidations of it to every arrival, which doubled the decode GEMMs' time (measured) and
  // orders nothing the write-through atomics do not already order.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(p.counters + t, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    s_flag = prev == S - 1;
  }
  __syncthreads();
  if (!s_flag) return;
  // last arrival: sum the partials in split order, the values of 4 splits in flight at a time
#pragma unroll
  for (int j = 0; j < T::NV; ++j) vals[j] = 0.f;
  for (int s0 = 0; owner && s0 < S; s0 += 4) {
    float v4[4][T::NV];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* src = base + ((size_t)t * S + min(s0 + u, S - 1)) * T::SLOT_FLOATS;
#pragma unroll
      for (int j = 0; j < T::NV; ++j)
        v4[u][j] = __hip_atomic_load(src + j * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < T::NV; ++j) vals[j] = s0 + u < S ? vals[j] + v4[u][j] : vals[j];
  }
  store_y();
  // re-arm for the next call (ordered before it by the kernel boundary)
  if (tid == 0)
    __hip_atomic_store(p.counters + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------------
// Decode-sized GEMM (M <= 4), weight streaming without any hand-off between workgroups.
// Workgroup t of 8 waves computes output columns [BN t, BN t + BN) (BN = 16 NB) for all M rows
// over the whole K range, which its waves split among themselves: wave w takes the K slices
// w, w + 8, w + 16, ... Each wave streams its slices' weight fragments (NB blocks of 16 rows x 128
// bytes), activation fragments (MT blocks of 16 rows) and scales straight from memory into a
// register ring D slices deep -- no LDS and no barrier inside the K loop, every load and wait
// visible to the compiler -- and multiplies each slice with the weight fragment as the matrix
// core's A operand (result rows = output columns) and the activation fragment as its B operand
// (result columns = output rows), so a lane's rescale needs one activation scale per row block.
// The eight partial tiles are then summed through LDS in wave order (the same bits every run)
// and stored.
// ---------------------------------------------------------------------------------------------
template <int MT_, int NB_, int D_>
struct Str {
  static constexpr int MT = MT_, NB = NB_, D = D_;
  static constexpr int WAVES = 8, NT = 512;
  static constexpr int BN = 16 * NB;
  static constexpr int PARTS = MT * NB;  // 16x16 blocks per wave
};

// One slice of a wave in registers. Unfused form: the activation codes and scales as stored by
// the 1x128 quantizer. Fused form (F, M <= kStrFusedRows): the slice's bf16 activation values
// instead, 8 per lane -- the 16 lanes of DPP row r hold row r's 1x128 group, so its amax is one
// row reduction -- quantized when the slice is multiplied.
constexpr int kStrFusedRows = 4;
constexpr int kStrRows = 4;  // the planner's streaming-kernel range (the fused form's as well)

template <class T, bool F>
struct StrSlot;

template <class T>
struct StrSlot<T, false> {
  v8i w[T::NB];
  v8i x[T::MT];
  float sa[T::MT];
  float sw;
};

template <class T>
struct StrSlot<T, true> {
  static_assert(T::MT == 1, "fused form: one 16-row block");
  v8i w[T::NB];
  u32x4 xb;
  float sw;
};

template <class T, bool F>
__device__ __forceinline__ void str_load(StrSlot<T, F>& s, const GemmArgs& p, int n0, int kb,
                                         int r16, int kq) {
#pragma unroll
  for (int j = 0; j < T::NB; ++j)
    s.w[j] = load_frag_global(p.wq + (int64_t)(n0 + 16 * j + r16) * p.K, kb, kq);
  if constexpr (F) {
    // lane l: values 8 (l % 16) .. + 7 of row l / 16 (rows past M repeat row M - 1)
    const int lane = 16 * kq + r16;
    const int m = min(lane >> 4, p.M - 1);
    s.xb = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * p.ld_x + (int64_t)kb * 128 +
                                           (lane & 15) * 8);
  } else {
#pragma unroll
    for (int i = 0; i < T::MT; ++i) {
      // rows past M repeat row M - 1: their products reach no stored output
      const int m = min(16 * i + r16, p.M - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(p.xq + (int64_t)m * p.K +
                                                        (int64_t)kb * 128 + kq * 32);
      const u32x4 lo = src[0], hi = src[1];
      s.x[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                   (int)hi.w};
      s.sa[i] = p.sa[(int64_t)m * p.KB + kb];
    }
  }
  s.sw = p.sw[(int64_t)(n0 >> 7) * p.KB + kb];
}

// Fused form: the 1x128 activation quantizer's arithmetic on one slice (the same amax, scale and
// element quotients, hence the same codes and scales), each of the M <= 4 live rows by one DPP
// row of 16 lanes -- so the work does not grow with the 16-row padding of the matrix-core
// operand. The codes and scales pass through this wave's own LDS area into the fragment layout
// (lane l: row l % 16, K quarter l / 16; rows past M read row M - 1). LDS accesses of one wave
// complete in order, so no barrier and no wait beyond the compiler's are needed.
template <class T>
__device__ __forceinline__ void str_quant(const StrSlot<T, true>& s, int M, int pow2,
                                          uint8_t* codes, float* scales, int r16, int kq,
                                          v8i (&xq)[1], float (&sa)[1]) {
  const int lane = 16 * kq + r16, row = lane >> 4, c = lane & 15;
  const uint32_t m = row16_max_u32(hmax_u16(amax8_pk(s.xb)));
  const float fs = scale_from_amax_bits(m), ps = pow2_scale_from_amax_bits(m);
  const float S = pow2 ? ps : fs;
  const u32x2 q = quant8(s.xb, recip_f64(S));
  if (row < M) {
    *reinterpret_cast<u32x2*>(codes + row * 128 + c * 8) = q;
    if (c == 0) scales[row] = S;
  }
  const int rr = min(r16, M - 1);
  const u32x4* src = reinterpret_cast<const u32x4*>(codes + rr * 128 + kq * 32);
  const u32x4 lo = src[0], hi = src[1];
  xq[0] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
              (int)hi.w};
  sa[0] = scales[rr];
}

template <class T, int ACC>
__device__ __forceinline__ void str_mma(const v8i (&w)[T::NB], const v8i (&x)[T::MT],
                                        const float (&sa)[T::MT], float sw,
                                        v4f (&acc)[T::MT][T::NB]) {
  if constexpr (ACC == 2) {
    const int swe = e8m0_of(sw);
#pragma unroll
    for (int i = 0; i < T::MT; ++i) {
      const int se = e8m0_of(sa[i]);
#pragma unroll
      for (int j = 0; j < T::NB; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[j], x[i], acc[i][j], 0,
                                                                     0, 0, swe, 0, se);
        asm volatile("" : "+v"(acc[i][j]));  // keep each slice's update in place
      }
    }
    return;
  }
  v4f pr[T::MT][T::NB];
#pragma unroll
  for (int i = 0; i < T::MT; ++i)
#pragma unroll
    for (int j = 0; j < T::NB; ++j) pr[i][j] = slice_product<ACC == 1>(w[j], x[i]);
  __builtin_amdgcn_sched_barrier(0);  // every product in flight before the first is consumed
#pragma unroll
  for (int i = 0; i < T::MT; ++i) {
    const float sc = sa[i] * sw;
#pragma unroll
    for (int j = 0; j < T::NB; ++j) {
      acc[i][j] += pr[i][j] * sc;
      asm volatile("" : "+v"(acc[i][j]));
    }
  }
}

// F: bf16 activations p.x (pitch p.ld_x, scale format p.pow2; M <= kStrFusedRows) quantized in
// the kernel instead of the codes p.xq and scales p.sa.
template <class T, int ACC, bool F>
__global__ __launch_bounds__(T::NT) void gemm_stream_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) v4f red[T::WAVES][T::PARTS][64];
  // fused form: each wave's staged codes (kStrFusedRows rows of one slice) and their scales
  __shared__ __attribute__((aligned(16))) uint8_t xcodes[F ? T::WAVES : 1][kStrFusedRows * 128];
  __shared__ float xscales[F ? T::WAVES : 1][kStrFusedRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * T::BN;
  const int KB = p.KB;
  // slices of this wave: wave + 8 t, t < cnt (cnt a multiple of D, the same for every wave)
  const int cnt = ((KB + T::WAVES - 1) / T::WAVES + T::D - 1) / T::D * T::D;
  v4f acc[T::MT][T::NB];
#pragma unroll
  for (int i = 0; i < T::MT; ++i)
#pragma unroll
    for (int j = 0; j < T::NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // The loop is free of branches, so that the compiler's wait counts stay exact (a slice's
  // operands are waited for with the D - 1 later slices still in flight): a slice past K is
  // loaded from the last slice and multiplied with zeroed activation codes, and the last round
  // (no refills) is peeled off.
  StrSlot<T, F> ring[T::D];
  auto mma = [&](StrSlot<T, F>& s, int kb) {
    if constexpr (F) {
      if (kb >= KB) s.xb = u32x4{0u, 0u, 0u, 0u};  // uniform: past K, zero codes and products
      v8i xq[1];
      float sa[1];
      str_quant<T>(s, p.M, p.pow2, xcodes[F ? wave : 0], xscales[F ? wave : 0], r16, kq, xq, sa);
      str_mma<T, ACC>(s.w, xq, sa, s.sw, acc);
    } else {
      if (kb >= KB) {  // uniform: past K, zero products
#pragma unroll
        for (int i = 0; i < T::MT; ++i) s.x[i] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
      str_mma<T, ACC>(s.w, s.x, s.sa, s.sw, acc);
    }
  };
#pragma unroll
  for (int u = 0; u < T::D; ++u)
    str_load<T, F>(ring[u], p, n0, min(wave + T::WAVES * u, KB - 1), r16, kq);
  for (int t = 0; t < cnt - T::D; t += T::D) {
#pragma unroll
    for (int u = 0; u < T::D; ++u) {
      mma(ring[u], wave + T::WAVES * (t + u));
      str_load<T, F>(ring[u], p, n0, min(wave + T::WAVES * (t + u + T::D), KB - 1), r16, kq);
    }
  }
#pragma unroll
  for (int u = 0; u < T::D; ++u) mma(ring[u], wave + T::WAVES * (cnt - T::D + u));
  // sum the eight waves' partial tiles in wave order
#pragma unroll
  for (int i = 0; i < T::MT; ++i)
#pragma unroll
    for (int j = 0; j < T::NB; ++j) red[wave][i * T::NB + j][lane] = acc[i][j];
  __syncthreads();
  for (int q = tid; q < T::PARTS * 64; q += T::NT) {
    const int part = q >> 6, l = q & 63;
    v4f s = red[0][part][l];
#pragma unroll
    for (int w = 1; w < T::WAVES; ++w) s += red[w][part][l];
    // block (i, j) = (part / NB, part % NB); lane l holds output row 16 i + l % 16 and the four
    // columns n0 + 16 j + 4 (l / 16) .. + 3
    const int m = 16 * (part / T::NB) + (l & 15);
    if (m >= p.M) continue;
    const int64_t off = (int64_t)m * p.ldy + n0 + 16 * (part % T::NB) + 4 * (l >> 4);
    if (p.out_f32) {
      *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.y) + off) = s;
    } else {
      const uint32_t lo = f32_to_bf16_rne(s[0]) | ((uint32_t)f32_to_bf16_rne(s[1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(s[2]) | ((uint32_t)f32_to_bf16_rne(s[3]) << 16);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.y) + off) = u32x2{lo, hi};
    }
  }
}

// Deterministic split-K reduction: partials are summed in split order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            int splits, int64_t M, int N, void* y,
                                                            int64_t ldy, int out_f32) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total4 = M * N / 4;
  if (i4 >= total4) return;
  const int64_t e = i4 * 4;
  const int64_t row = e / N, col = e - (e / N) * N;
  float4 s = reinterpret_cast<const float4*>(ws)[i4];
  for (int k = 1; k < splits; ++k) {
    const float4 t = reinterpret_cast<const float4*>(ws + (int64_t)k * M * N)[i4];
    s.x += t.x;
    s.y += t.y;
    s.z += t.z;
    s.w += t.w;
  }
  if (out_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + row * ldy + col) = s;
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(y) + row * ldy + col;
    const uint32_t lo = f32_to_bf16_rne(s.x) | ((uint32_t)f32_to_bf16_rne(s.y) << 16);
    const uint32_t hi = f32_to_bf16_rne(s.z) | ((uint32_t)f32_to_bf16_rne(s.w) << 16);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------------------------
// Grouped GEMM. The grid enumerates (m-tile, n-tile) pairs up to the bound
// sum_e ceil(rows_e / BM) <= M_total / BM + E; each workgroup reads the offsets, forms the
// per-expert tile counts and their prefix sums in LDS, finds which expert its m-tile belongs to
// and exits if it is past the last real tile. No host round trip and no workspace are needed.
// ---------------------------------------------------------------------------------------------

template <class T, bool PRECISE>
__global__ __launch_bounds__(T::NT) void grouped_gemm_kernel(GemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_scan = reinterpret_cast<int*>(smem + T::LDS_BYTES);  // [NT] scan scratch
  __shared__ int s_expert, s_row0, s_rows;

  const int tid = threadIdx.x;
  const int tm_lin = blockIdx.x / p.tiles_n;
  const int tn = blockIdx.x - tm_lin * p.tiles_n;

  if (tid == 0) s_expert = -1;
  // exclusive scan of per-expert m-tile counts, NT experts per pass, carried across passes
  int carry = 0;
  for (int base = 0; base < p.E; base += T::NT) {
    const int e = base + tid;
    int lo = 0, hi = 0, cnt = 0;
    if (e < p.E) {
      lo = min(max(p.offsets[e], 0), p.M);
      hi = min(max(p.offsets[e + 1], lo), p.M);
      cnt = (hi - lo + T::BM - 1) / T::BM;
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < T::NT; d <<= 1) {
      const int v = tid >= d ? s_scan[tid - d] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int incl = s_scan[tid] + carry;
    const int excl = incl - cnt;
    if (e < p.E && cnt > 0 && tm_lin >= excl && tm_lin < incl) {
      s_expert = e;
      s_row0 = lo + (tm_lin - excl) * T::BM;
      s_rows = min(T::BM, hi - s_row0);
    }
    carry += s_scan[T::NT - 1];
    __syncthreads();
  }
  const int e = s_expert;
  if (e < 0) return;  // past the last real tile (uniform across the workgroup)
  const int row0 = s_row0, m_valid = s_rows;
  const int n0 = tn * T::BN;
  v4f acc[T::TM][T::TN];
  run_tile<T, PRECISE>(p.xq + (int64_t)row0 * p.K, p.sa + (int64_t)row0 * p.KB, m_valid,
              p.wq + e * p.wq_stride + (int64_t)n0 * p.K, p.sw + e * p.sw_stride, n0, T::BN, p.K,
              p.KB, 0, p.KB, smem, acc);
  store_tile<T>(p, row0, m_valid, n0, 0, acc);
}

// ---------------------------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr int kCfgLarge = 0, kCfgSmall = 1, kCfgBigWide = 2, kCfgBigNarrow = 3, kCfgDecode = 4,
              kCfgGroupedBig = 5, kCfgStream = 6;
constexpr int64_t kGroupedWorkgroups = 256;  // persistent grouped GEMM: one per CU (LDS-bound)
constexpr int kTargetWorkgroups = 512;  // two per CU on 256 CUs
constexpr int kMinSlicesPerSplit = 4;

// Kernels that use more than the default 64 KiB of dynamic LDS must opt in, once per kernel and
// device. `done` holds one bit per device id (ids >= 64 always call the runtime).
hipError_t ensure_lds(std::atomic<uint64_t>& done, const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool rowb) {
  GemmPlan pl{};
  const int64_t KB = K / 128;
  // the DMA-fed 256-row tiles also from 192 rows on, once the 256 x 128 tiles alone number
  // at least 128 (half a wave of workgroups over the chip): below 1024 rows the 64 x 64 tiles'
  // extra operand traffic costs more than the padded rows of a part-filled 256-row tile
  const int64_t narrow_tiles = ((M + 255) / 256) * (N / 128);
  if ((M >= 1024 || (M >= 192 && narrow_tiles >= 128)) && KB <= kMaxSlices) {
    const int64_t wide_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    pl.cfg = wide_tiles >= 240 ? kCfgBigWide : kCfgBigNarrow;
    pl.bm = 256;
    pl.bn = pl.cfg == kCfgBigWide ? 256 : 128;
    pl.splits = 1;
    pl.kb_per_split = (int)KB;
    pl.workspace_bytes = 0;
    return pl;
  }
  if (M <= kStrRows && !rowb) {
    // weight streaming, K split over the waves of each workgroup (no workspace). Each
    // workgroup reads all M activation rows for its 16 or 32 columns; on the Qwen3-8B decode
    // GEMMs (graph-replayed) it beats the split-K decode GEMM below up to 4 rows (51.3 against
    // 57.8 us for the four GEMMs at M = 1) and loses from 8 rows on (60.7 / 58.0 us at M = 8,
    // 67.0 / 58.2 us at M = 16), as its activation reads grow with M.
    pl.cfg = kCfgStream;
    pl.bm = 16;
    pl.bn = N % 32 == 0 && N / 16 > 1024 ? 32 : 16;
    const int64_t per_wave = (KB + 7) / 8;  // slices per wave
    pl.depth = per_wave >= 4 ? 4 : 2;
    pl.splits = 1;
    pl.kb_per_split = (int)KB;
    pl.workspace_bytes = 0;
    return pl;
  }
  if (M <= 64 && !rowb) return plan_decode(M, N, K);  // the split-K decode GEMM
  // 64 x 64 tiles below 1024 rows: against 128 x 128 tiles split four ways over K they measured
  // 1.3-2x faster at 512-1000 rows (the split partials' round trip through memory outweighs the
  // larger tile's operand reuse); the 128 x 128 tiles stay for K beyond the DMA-fed tiles' reach
  if (M >= 1024) {
    pl.cfg = kCfgLarge;
    pl.bm = TileLarge::BM;
    pl.bn = TileLarge::BN;
  } else {
    pl.cfg = kCfgSmall;
    pl.bm = TileSmall::BM;
    pl.bn = TileSmall::BN;
  }
  const int64_t tiles = ((M + pl.bm - 1) / pl.bm) * (N / pl.bn);
  int64_t splits = 1;
  if (tiles > 0 && tiles < kTargetWorkgroups) {
    splits = (kTargetWorkgroups + tiles - 1) / tiles;
    const int64_t max_splits = KB / kMinSlicesPerSplit;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
  }
  pl.kb_per_split = (int)((KB + splits - 1) / splits);
  pl.splits = (int)((KB + pl.kb_per_split - 1) / pl.kb_per_split);
  if (pl.splits < 1) pl.splits = 1;
  pl.workspace_bytes =
      pl.splits > 1 ? kWsHeaderBytes + (size_t)pl.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
  return pl;
}

GemmPlan plan_decode(int64_t M, int64_t N, int64_t K) {
  GemmPlan pl{};
  const int64_t KB = K / 128;
  // 5 <= M <= 64 (rows padded to 32 or 64). Tiles of 64 columns; while they number at most 256,
  // two K halves per workgroup (8 waves, one workgroup per CU) and K split into S ranges, S the
  // largest power of two that keeps the grid within one round of 256 workgroups and each range
  // at least 4 slices; past 256 tiles one K half and S = 1 (2 up to 32 rows, where the
  // partials are half as large). Wide GEMMs above 32 rows: 128-column tiles (half the
  // activation bytes per weight byte) with two K halves and no split. Measured on the Qwen3-8B
  // decode GEMMs at M = 64 (graph-replayed, weights rotated), two halves against one: gate/up
  // 24576x4096 26.6 against 30.2 us (128 columns, unsplit), o 4096x4096 8.9 against 10.0 us and
  // down 4096x12288 18.1 against 20.4 us (S = 4), q/k/v 6144x4096 10.8 us either way (S = 2
  // against 4); with more workgroups than CUs two halves lose (q/k/v at S = 4: 13.2 us).
  const int64_t bm = M <= 32 ? 32 : 64;
  int64_t BN = 64, S = 1, KH = KB >= 4 ? 2 : 1;
  if (M > 32 && N / 128 >= 192) {
    BN = 128;
    if (N / 128 > 256) KH = 1;
  } else {
    const int64_t tiles = N / 64;
    if (tiles <= 256) {
      while (tiles * 2 * S <= 256 && KB / (2 * S) >= 4) S *= 2;
    } else {
      KH = 1;
      if (M <= 32 && KB >= 8) S = 2;
    }
    if (tiles > kWsCounters) S = 1;
  }
  const int64_t tiles = N / BN;
  const int64_t L = (KB + S - 1) / S;
  S = (KB + L - 1) / L;  // no empty range
  pl.cfg = kCfgDecode;
  pl.bm = BN == 128 ? 64 : (int)bm;  // the 128-column tile is built for 64 rows
  pl.bn = (int)BN;
  pl.depth = (int)KH;  // K halves per workgroup
  pl.splits = (int)S;
  pl.kb_per_split = (int)L;
  pl.workspace_bytes = S > 1 ? kWsHeaderBytes + (size_t)(tiles * S) * BN * pl.bm * sizeof(float) : 0;
  return pl;
}

GemmPlan plan_fused_act(int64_t M, int64_t N, int64_t K) {
  GemmPlan pl = plan_gemm(M, N, K);
  // up to kStrFusedRows rows the streaming kernel quantizes the activations itself (one launch,
  // no workspace). Every workgroup quantizes all of X again, which pays only while that work is
  // small against the weight stream: with 16 rows the fused streaming kernel took 1.2x as long as
  // two launches, and with 64 rows a form of the decode GEMM that quantizes each slice's bf16
  // rows in LDS took 2.1x (every activation group quantized once per 64-column tile and split,
  // with float64 quotients). Above, the codes and
  // scales are staged in the workspace by the 1x128 quantizer and the GEMM of the same plan
  // reads them: [GEMM workspace | codes | scales], each part 256-byte aligned. The counter header
  // stays reserved even where this GEMM splits nothing, so that the workspace keeps it zero.
  if (pl.cfg == kCfgStream && M <= kStrFusedRows) return pl;
  const size_t a256 = 255;
  pl.stage_off = std::max((pl.workspace_bytes + a256) & ~a256, kWsHeaderBytes);
  const size_t codes = ((size_t)M * (size_t)K + a256) & ~a256;
  pl.workspace_bytes = pl.stage_off + codes + (size_t)M * (size_t)(K / 128) * sizeof(float);
  return pl;
}

GemmPlan plan_grouped_fused_act(int64_t M, int64_t N, int64_t K, int32_t E) {
  // [counter header, kept zero | codes of M rows | their scales] and, where the grouped GEMM
  // runs on the register-staged tiles (no row gather there), a second such area for the
  // gathered rows; each part 256-byte aligned
  GemmPlan pl = plan_grouped_gemm(M, N, K, E);
  const size_t a256 = 255;
  const size_t area = (((size_t)M * (size_t)K + a256) & ~a256) +
                      (((size_t)M * (size_t)(K / 128) * sizeof(float) + a256) & ~a256);
  pl.stage_off = kWsHeaderBytes;
  pl.workspace_bytes = kWsHeaderBytes + (pl.cfg == kCfgGroupedBig ? 1 : 2) * area;
  return pl;
}

GemmPlan plan_grouped_gemm(int64_t M_total, int64_t N, int64_t K, int32_t E) {
  GemmPlan pl{};
  (void)M_total;
  (void)E;
  const bool big = K / 128 <= kMaxSlices;
  pl.cfg = big ? kCfgGroupedBig : kCfgLarge;
  pl.bm = big ? BigGroup::BM : TileLarge::BM;
  pl.bn = big ? BigGroup::BN : TileLarge::BN;
  pl.splits = big ? (int)kGroupedWorkgroups : 1;  // persistent workgroups
  pl.kb_per_split = (int)(K / 128);
  pl.workspace_bytes = 0;
  return pl;
}

template <class T, int ACC>
static hipError_t launch_big(const GemmArgs& a, hipStream_t stream) {
  const int tiles_m = (a.M + T::BM - 1) / T::BM;
  const int tiles_n = (a.N + T::BN - 1) / T::BN;
  hipLaunchKernelGGL((gemm_big_kernel<T, ACC>), dim3((unsigned)(tiles_m * tiles_n)), dim3(T::NT),
                     0, stream, a);
  return hipGetLastError();
}

template <class T, int ACC, bool F>
static hipError_t launch_stream_t(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_stream_kernel<T, ACC, F>), dim3((unsigned)(a.N / T::BN)), dim3(T::NT),
                     0, stream, a);
  return hipGetLastError();
}

template <int MT, int NB, int ACC, bool F>
static hipError_t launch_stream_d(const GemmArgs& a, const GemmPlan& pl, hipStream_t stream) {
  if (pl.depth == 4) return launch_stream_t<Str<MT, NB, 4>, ACC, F>(a, stream);
  return launch_stream_t<Str<MT, NB, 2>, ACC, F>(a, stream);
}

template <int ACC, bool F = false>
static hipError_t launch_stream(const GemmArgs& a, const GemmPlan& pl, hipStream_t stream) {
  if (pl.bn == 32) return launch_stream_d<1, 2, ACC, F>(a, pl, stream);
  return launch_stream_d<1, 1, ACC, F>(a, pl, stream);
}

template <class T, int ACC>
static hipError_t launch_decode_t(const GemmArgs& a, const GemmPlan& pl, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_decode_kernel<T, ACC>),
                     dim3((unsigned)(a.N / T::BN), (unsigned)pl.splits), dim3(T::NT), 0, stream, a);
  return hipGetLastError();
}

template <int ACC, int KH>
static hipError_t launch_decode_k(const GemmArgs& a, const GemmPlan& pl, hipStream_t stream) {
  if (pl.bn == 128) return launch_decode_t<Dec<64, 128, 32, KH>, ACC>(a, pl, stream);  // M > 32
  return pl.bm == 32 ? launch_decode_t<Dec<32, 64, 16, KH>, ACC>(a, pl, stream)
                     : launch_decode_t<Dec<64, 64, 16, KH>, ACC>(a, pl, stream);
}

template <int ACC>
static hipError_t launch_decode(const GemmArgs& a, const GemmPlan& pl, hipStream_t stream) {
  return pl.depth == 2 ? launch_decode_k<ACC, 2>(a, pl, stream) : launch_decode_k<ACC, 1>(a, pl, stream);
}

template <class T, bool PRECISE>
static hipError_t launch_dense(const GemmArgs& a, const GemmPlan& pl, hipStream_t stream) {
  static std::atomic<uint64_t> lds_done{0};
  hipError_t e = ensure_lds(lds_done, (const void*)gemm_kernel<T, PRECISE>, T::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int tiles_m = (a.M + T::BM - 1) / T::BM;
  const int tiles_n = a.N / T::BN;
  dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)pl.splits);
  hipLaunchKernelGGL((gemm_kernel<T, PRECISE>), grid, dim3(T::NT), T::LDS_BYTES, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, void* y, int out_f32, int64_t ld_y,
                       int accum, int rowb, void* workspace, const GemmPlan& pl,
                       hipStream_t stream) {
  // accum: 0 FP8 slice sums, 1 f16 slice sums, 2 power-of-two scales in the matrix cores (the
  // register-staged tiles have no such form: their FP8 form gives the same results then)
  const bool precise = accum == 1;
  GemmArgs a{};
  a.xq = xq;
  a.sa = sa;
  a.wq = wq;
  a.sw = sw;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.KB = (int)(K / 128);
  a.y = y;
  a.ldy = ld_y;
  a.out_f32 = out_f32;
  // workspace: the counter header, then the partials
  a.counters = pl.workspace_bytes > 0 ? reinterpret_cast<int*>(workspace) : nullptr;
  a.ws = pl.workspace_bytes > 0
             ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kWsHeaderBytes)
             : nullptr;
  a.splits = pl.splits;
  a.kb_per_split = pl.kb_per_split;
  hipError_t e;
  if (rowb) {  // sw is sb [N][KB]: one scale per B row and slice
    switch (pl.cfg) {
      case kCfgBigWide:
        if (accum == 1) return launch_big<BigF16Row, 1>(a, stream);
        return accum == 2 ? launch_big<BigWideRow, 2>(a, stream) : launch_big<BigWideRow, 0>(a, stream);
      case kCfgBigNarrow:
        if (accum == 1) return launch_big<BigF16Row, 1>(a, stream);
        return accum == 2 ? launch_big<BigNarrowRow, 2>(a, stream)
                          : launch_big<BigNarrowRow, 0>(a, stream);
      case kCfgLarge:
        e = precise ? launch_dense<TileLargeRow, true>(a, pl, stream)
                    : launch_dense<TileLargeRow, false>(a, pl, stream);
        break;
      default:  // the planner never picks the decode path for row-scaled B
        e = precise ? launch_dense<TileSmallRow, true>(a, pl, stream)
                    : launch_dense<TileSmallRow, false>(a, pl, stream);
        break;
    }
  } else {
  switch (pl.cfg) {
    case kCfgBigWide:
      // the f16 form needs more registers per wave than the 8-wave 256x256 tile leaves
      if (accum == 1) return launch_big<BigF16, 1>(a, stream);
      return accum == 2 ? launch_big<BigWide, 2>(a, stream) : launch_big<BigWide, 0>(a, stream);
    case kCfgBigNarrow:
      if (accum == 1) return launch_big<BigF16, 1>(a, stream);
      return accum == 2 ? launch_big<BigNarrow, 2>(a, stream) : launch_big<BigNarrow, 0>(a, stream);
    case kCfgStream:
      if (accum == 1) return launch_stream<1>(a, pl, stream);
      return accum == 2 ? launch_stream<2>(a, pl, stream) : launch_stream<0>(a, pl, stream);
    case kCfgDecode:  // reduces its own split tiles
      if (accum == 1) return launch_decode<1>(a, pl, stream);
      return accum == 2 ? launch_decode<2>(a, pl, stream) : launch_decode<0>(a, pl, stream);
    case kCfgLarge:
      e = precise ? launch_dense<TileLarge, true>(a, pl, stream)
                  : launch_dense<TileLarge, false>(a, pl, stream);
      break;
    default:
      e = precise ? launch_dense<TileSmall, true>(a, pl, stream)
                  : launch_dense<TileSmall, false>(a, pl, stream);
      break;
  }
  }
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t total4 = M * N / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0,
                     stream, a.ws, pl.splits, M, (int)N, y, ld_y, out_f32);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Scratch for the no-allocation entry point: one static device array per device (the code
// object's copy on each device it is loaded on), used exactly like a caller's workspace --
// arrival counters in the first kWsHeaderBytes, split partials after them. In host code the
// array's name is only a stand-in; its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is ever passed to kernels.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

}  // namespace

hipError_t gemm_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the counters must start at zero (the loader zero-fills the array too); every GEMM that
    // uses them leaves them zero again. A fill kernel, not a memset, so that a caller may
    // capture this first call into a graph.
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(p), (int)(kWsHeaderBytes / 4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gemm_fused_act(const uint16_t* x, int64_t ld_x, int pow2, const uint8_t* wq,
                                 const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                 int out_f32, int64_t ld_y, int accum, void* workspace,
                                 const GemmPlan& pl, hipStream_t stream) {
  if (pl.cfg == kCfgStream && M <= kStrFusedRows) {
    GemmArgs a{};
    a.x = x;
    a.ld_x = ld_x;
    a.pow2 = pow2;
    a.wq = wq;
    a.sw = sw;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.KB = (int)(K / 128);
    a.y = y;
    a.ldy = ld_y;
    a.out_f32 = out_f32;
    a.splits = 1;
    a.kb_per_split = a.KB;
    if (accum == 1) return launch_stream<1, true>(a, pl, stream);
    return accum == 2 ? launch_stream<2, true>(a, pl, stream) : launch_stream<0, true>(a, pl, stream);
  }
  // staged: quantize into the workspace behind the GEMM's own part, then the GEMM on the codes
  uint8_t* xq = reinterpret_cast<uint8_t*>(workspace) + pl.stage_off;
  float* sa = reinterpret_cast<float*>(xq + ((((size_t)M * (size_t)K) + 255) & ~size_t{255}));
  hipError_t e = launch_quant_act(x, M, K, ld_x, xq, K, sa, pow2, stream);
  if (e != hipSuccess) return e;
  // the GEMM's own plan: its workspace size alone decides whether it splits K
  return launch_gemm(xq, sa, wq, sw, M, N, K, y, out_f32, ld_y, accum, 0, workspace,
                     plan_gemm(M, N, K), stream);
}

hipError_t launch_grouped_gemm(const uint8_t* xq, const float* sa, const uint8_t* wq,
                               const float* sw, const int32_t* offsets, int32_t E,
                               int64_t M_total, int64_t N, int64_t K, void* y, int out_f32,
                               int accum, void* workspace, const GemmPlan& pl,
                               hipStream_t stream, const int32_t* rows, int64_t src_rows) {
  (void)workspace;
  if (rows && pl.cfg != kCfgGroupedBig) return hipErrorInvalidValue;  // gather: DMA-fed tiles only
  const bool precise = accum == 1;
  using T = TileLarge;
  GemmArgs a{};
  a.xq = xq;
  a.sa = sa;
  a.wq = wq;
  a.sw = sw;
  a.M = (int)M_total;
  a.N = (int)N;
  a.K = (int)K;
  a.KB = (int)(K / 128);
  a.y = y;
  a.ldy = N;
  a.out_f32 = out_f32;
  a.ws = nullptr;
  a.splits = 1;
  a.kb_per_split = a.KB;
  a.offsets = offsets;
  a.E = E;
  a.wq_stride = N * K;
  a.sw_stride = (N / 128) * (K / 128);
  a.rows = rows;
  a.src_rows = (int)src_rows;
  if (pl.cfg == kCfgGroupedBig) {
    a.tiles_n = (int)((N + BigGroup::BN - 1) / BigGroup::BN);
    const dim3 grid((unsigned)pl.splits), block(BigGroup::NT);
    if (accum == 1)
      hipLaunchKernelGGL((grouped_big_kernel<BigGroup, 1>), grid, block, 0, stream, a);
    else if (accum == 2)
      hipLaunchKernelGGL((grouped_big_kernel<BigGroup, 2>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((grouped_big_kernel<BigGroup, 0>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  a.tiles_n = (int)(N / T::BN);
  const int lds = T::LDS_BYTES + T::NT * (int)sizeof(int);
  static std::atomic<uint64_t> lds_done_fast{0}, lds_done_precise{0};
  const void* kern = precise ? (const void*)grouped_gemm_kernel<T, true>
                             : (const void*)grouped_gemm_kernel<T, false>;
  hipError_t e = ensure_lds(precise ? lds_done_precise : lds_done_fast, kern, lds);
  if (e != hipSuccess) return e;
  // sum_e ceil(rows_e / BM) <= sum_e (rows_e / BM + 1) <= ceil(M_total / BM) + E
  const int64_t tiles_m_bound = (M_total + T::BM - 1) / T::BM + E;
  const int64_t grid = tiles_m_bound * a.tiles_n;
  if (precise)
    hipLaunchKernelGGL((grouped_gemm_kernel<T, true>), dim3((unsigned)grid), dim3(T::NT), lds,
                       stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<T, false>), dim3((unsigned)grid), dim3(T::NT), lds,
                       stream, a);
  return hipGetLastError();
}

// Copy the codes and scales of source rows rows[r] (clamped to [0, src_rows - 1]) to row r,
// r < M: a workgroup per row (grid-stride), 16-byte pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ xq,
                                                          const float* __restrict__ sa,
                                                          const int32_t* __restrict__ rows,
                                                          int src_rows, int64_t M, int K,
                                                          uint8_t* out_q, float* out_s) {
  const int KB = K / 128;
  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    const int64_t src = min(max(rows[r], 0), src_rows - 1);
    for (int c = threadIdx.x; c < K / 16; c += 256)
      reinterpret_cast<uint4*>(out_q + r * K)[c] = reinterpret_cast<const uint4*>(xq + src * K)[c];
    for (int c = threadIdx.x; c < KB; c += 256) out_s[r * KB + c] = sa[src * KB + c];
  }
}

hipError_t launch_grouped_gemm_fused_act(const uint16_t* x, int64_t ld_x, int64_t src_rows,
                                         const int32_t* rows, int pow2, const uint8_t* wq,
                                         const float* sw, const int32_t* offsets, int32_t E,
                                         int64_t M_total, int64_t N, int64_t K, void* y,
                                         int out_f32, int accum, void* workspace,
                                         hipStream_t stream) {
  const int64_t M = rows ? src_rows : M_total;
  const GemmPlan pl = plan_grouped_fused_act(std::max(src_rows, M_total), N, K, E);
  const size_t a256 = 255;
  const int64_t KB = K / 128;
  auto codes_of = [&](size_t off) { return reinterpret_cast<uint8_t*>(workspace) + off; };
  auto scales_of = [&](size_t off, int64_t m) {
    return reinterpret_cast<float*>(codes_of(off) + (((size_t)m * (size_t)K + a256) & ~a256));
  };
  // each source row once, into the first area
  uint8_t* xq = codes_of(pl.stage_off);
  float* sa = scales_of(pl.stage_off, M);
  hipError_t e = launch_quant_act(x, M, K, ld_x, xq, K, sa, pow2, stream);
  if (e != hipSuccess) return e;
  const GemmPlan gp = plan_grouped_gemm(M_total, N, K, E);
  if (rows && gp.cfg != kCfgGroupedBig) {
    // the register-staged tiles read contiguous rows: gather them into the second area
    const size_t off2 = pl.stage_off + (((size_t)M * (size_t)K + a256) & ~a256) +
                        (((size_t)M * (size_t)KB * sizeof(float) + a256) & ~a256);
    uint8_t* xg = codes_of(off2);
    float* sg = scales_of(off2, M_total);
    const int64_t wgs = std::min<int64_t>(M_total, 16384);
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, xq, sa, rows,
                       (int)src_rows, M_total, (int)K, xg, sg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_grouped_gemm(xg, sg, wq, sw, offsets, E, M_total, N, K, y, out_f32, accum,
                               nullptr, gp, stream, nullptr, 0);
  }
  return launch_grouped_gemm(xq, sa, wq, sw, offsets, E, M_total, N, K, y, out_f32, accum, nullptr,
                             gp, stream, rows, src_rows);
}

}  // namespace fp8rl
