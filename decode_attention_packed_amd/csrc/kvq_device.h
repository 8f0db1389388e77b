// Device-side helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kBlock = 32;   // elements per quantization block along head_dim
constexpr int kTile = 32;    // tokens per V tile (V is stored token-interleaved per tile)
constexpr int kRows = 16;    // MFMA rows: query tokens x query heads of one kv group, padded

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// fp32 -> binary16 bits with the hardware conversion (round to nearest even,
// binary16 subnormals kept).
__device__ __forceinline__ uint16_t f32_to_half_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Integer code of x for scale d: the fp32 quotient (correctly rounded
// division), rounded to nearest even, clamped to [lo, hi]; 0 when d == 0.
__device__ __forceinline__ int quant_code(float x, float d, float lo, float hi) {
  if (d == 0.0f) return 0;
  float r = rintf(x / d);
  return (int)fminf(fmaxf(r, lo), hi);
}

// Cross-lane moves.  DPP controls (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1
// (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2), row_half_mirror = 0x141
// (lane i <-> 7-i inside each 8), row_mirror = 0x140 (lane i <-> 15-i inside
// each 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

// Exchanges between rows of 16 lanes without LDS (gfx950 lane swaps).  With
// both registers holding x, v_permlane16_swap leaves x of the even rows in the
// first and x of the odd rows in the second, in every lane, so combining the
// two applies op to (x, x ^ 16); v_permlane32_swap does the same for the two
// halves of the wave, (x, x ^ 32).  Issued from inline assembly: the
// compiler's builtin for these swaps reads the first result's register for
// both results once they meet in one arithmetic operation.  The s_nop covers
// the wait states between a VALU write and the swap's read.
template <class Op>
__device__ __forceinline__ float across16(float x, Op op) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(a, b);
}
template <class Op>
__device__ __forceinline__ float across32(float x, Op op) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(a, b);
}
__device__ __forceinline__ float fadd(float a, float b) { return a + b; }
__device__ __forceinline__ float fmax2(float a, float b) { return fmaxf(a, b); }

// Max / sum over the 16 lanes of a DPP row (lane ^ 1, ^ 2, mirror in 8, mirror in 16).
__device__ __forceinline__ float max_row16(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return x;
}
__device__ __forceinline__ float sum_row16(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}

// Max / min over the 32 lanes of a half-wave: DPP inside each 16-lane row,
// then one exchange between the two rows.
__device__ __forceinline__ float half_max(float x) {
  return across16(max_row16(x), fmax2);
}
// Max / sum over all 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_max(float x) {
  return across32(across16(max_row16(x), fmax2), fmax2);
}
__device__ __forceinline__ float wave_sum(float x) {
  return across32(across16(sum_row16(x), fadd), fadd);
}
__device__ __forceinline__ int half_min(int x) {
  x = min(x, dpp_i<0xB1>(x));
  x = min(x, dpp_i<0x4E>(x));
  x = min(x, dpp_i<0x141>(x));
  x = min(x, dpp_i<0x140>(x));
  return min(x, __shfl_xor(x, 16));
}

// Block quantization of the cache formats (page 1: int8 K payload with an
// fp16 scale per 32-block; V as q4_0 or q8_0).  The 32 lanes of a half-wave
// hold the 32 elements of one block, lane e element e.
//
// Symmetric int8 (K and q8_0 V): a = max|x|, d = fp16(a / 127),
// c = clamp(rne(x / d), -127, 127).  Returns the scale bits.
__device__ __forceinline__ uint16_t quant_sym8(float x, int& code) {
  const float a = half_max(fabsf(x));
  const uint16_t dbits = f32_to_half_bits(a / 127.0f);
  const float d = half_bits_to_f32(dbits);
  code = quant_code(x, d, -127.0f, 127.0f);
  return dbits;
}

// q4_0: m = first element of largest magnitude, d = fp16(m / -8),
// n = clamp(rne(x / d) + 8, 0, 15).  Returns the scale bits; `byte` is
// n_e | n_{e+16} << 4, the block's byte e, on lanes e < 16.
__device__ __forceinline__ uint16_t quant_q4_0(float x, int e, uint32_t& byte) {
  const float ax = fabsf(x);
  const float a = half_max(ax);
  const int first = half_min(ax == a ? e : kBlock);
  const float m = __shfl(x, ((int)__lane_id() & 32) + first);
  // fp16(m / -8) of m = +-0 is -+0.  The compiler contracts the scaling and
  // the fp16 conversion into one fma with a +0 addend, which would turn -0
  // into +0, so the zero case is spelled out.
  const uint16_t dbits = (m == 0.0f) ? (signbit(m) ? (uint16_t)0x0000 : (uint16_t)0x8000)
                                     : f32_to_half_bits(m / -8.0f);
  const float d = half_bits_to_f32(dbits);
  const int n = quant_code(x, d, -8.0f, 7.0f) + 8;
  const int n_hi = __shfl_xor(n, 16);
  byte = (uint32_t)(n | (n_hi << 4));
  return dbits;
}

// One element of Q quantization: x is element `idx` of a row of blocks, and
// the 32 lanes of this half-wave hold the 32 elements of its block.  Per
// 32-block a = max|x|, d = a / 127 kept in fp32, codes as quant_code.
__device__ __forceinline__ void quantize_q_lane(float x, int idx, int8_t* codes, float* scales) {
  const float a = half_max(fabsf(x));
  const float d = a / 127.0f;
  codes[idx] = (int8_t)quant_code(x, d, -127.0f, 127.0f);
  if ((idx & 31) == 0) scales[idx / kBlock] = d;
}

// Quantize `n` (a multiple of 64) consecutive fp32 values of Q with one wave.
// Codes go to `codes` (n bytes) and scales to `scales` (n / 32 floats); both
// may be LDS or global.  Lanes 0..31 and 32..63 each cover one block per step.
__device__ __forceinline__ void quantize_q_wave(const float* src, int n, int8_t* codes,
                                                float* scales) {
  const int lane = __lane_id();
  for (int e0 = 0; e0 < n; e0 += 64) quantize_q_lane(src[e0 + lane], e0 + lane, codes, scales);
}

// Segment lookup for token t of sequence `seq`.
__device__ __forceinline__ int segment_of(const int32_t* seg_table, int seq, int max_segs,
                                          int segj) {
  return seg_table ? seg_table[seq * max_segs + segj] : seq * max_segs + segj;
}

}  // namespace kvq
