// kv_append_quant kernel: quantize and pack new K/V rows into the cache.
//
// Page 1 ("Flash Attention for llama.cpp on RDNA3 ... Part 1", summary and
// first body paragraph): each new K row is re-packed on the fly to int8
// codes, four per 32-bit word, with an fp16 scale per 32-block; V is written
// as q4_0 or q8_0 blocks.  One thread owns one 32-block of one row and
// writes K (8 words + scale) and V (16 or 32 bytes + scale) for it.

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

struct AppendParams {
  const float* k_new;
  const float* v_new;
  uint32_t* k_qs;
  uint16_t* k_d;
  uint8_t* v_qs;
  uint16_t* v_d;
  const int32_t* seg_table;
  const int32_t* start_pos;
  int n_rows;        // n_seq * n_new * n_kv_heads
  int n_new;
  int n_kv_heads;
  int head_dim;
  int seg_tokens;
  int max_segs;
  int v_format;
};

__global__ __launch_bounds__(256) void k_append_quant(AppendParams p) {
  const int nb = p.head_dim / kBlock;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= p.n_rows * nb) return;
  const int row = gid / nb;
  const int b = gid - row * nb;
  const int h = row % p.n_kv_heads;
  const int j = (row / p.n_kv_heads) % p.n_new;
  const int seq = row / (p.n_kv_heads * p.n_new);

  const int pos = p.start_pos[seq] + j;
  const int segj = pos / p.seg_tokens;
  const int seg = segment_of(p.seg_table, seq, p.max_segs, segj);
  const size_t crow = ((size_t)seg * p.n_kv_heads + h) * p.seg_tokens + (pos - segj * p.seg_tokens);

  float x[kBlock];

  // ---- K: a = max|x|, d = fp16(a / 127), codes with the fp16 scale
  {
    const float4* src = reinterpret_cast<const float4*>(p.k_new + (size_t)row * p.head_dim + b * kBlock);
#pragma unroll
    for (int i = 0; i < kBlock / 4; ++i) {
      float4 v = src[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) a = fmaxf(a, fabsf(x[i]));
    const uint16_t dbits = f32_to_half_bits(a / 127.0f);
    const float d = half_bits_to_f32(dbits);
    uint32_t w[kBlock / 4];
#pragma unroll
    for (int i = 0; i < kBlock / 4; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        word |= ((uint32_t)(quant_code(x[4 * i + k], d, -127.0f, 127.0f) & 0xFF)) << (8 * k);
      w[i] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(p.k_qs + crow * (p.head_dim / 4) + b * (kBlock / 4));
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    p.k_d[crow * nb + b] = dbits;
  }

  // ---- V
  {
    const float4* src = reinterpret_cast<const float4*>(p.v_new + (size_t)row * p.head_dim + b * kBlock);
#pragma unroll
    for (int i = 0; i < kBlock / 4; ++i) {
      float4 v = src[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
    if (p.v_format == 0) {
      // q4_0: m = first element of largest magnitude, d = fp16(m / -8),
      // n = clamp(rne(x/d) + 8, 0, 15); byte j = n_j | n_{j+16} << 4
      float a = -1.0f, m = 0.0f;
#pragma unroll
      for (int i = 0; i < kBlock; ++i) {
        const float ax = fabsf(x[i]);
        if (ax > a) { a = ax; m = x[i]; }
      }
      // fp16(m / -8) of m = +-0 is -+0.  The compiler contracts the scaling
      // and the fp16 conversion into one fma with a +0 addend, which would
      // turn -0 into +0, so the zero case is spelled out.
      const uint16_t dbits = (m == 0.0f) ? (signbit(m) ? (uint16_t)0x0000 : (uint16_t)0x8000)
                                         : f32_to_half_bits(m / -8.0f);
      const float d = half_bits_to_f32(dbits);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int jj = 4 * i + k;
          const uint32_t lo = (d == 0.0f) ? 8u : (uint32_t)(quant_code(x[jj], d, -8.0f, 7.0f) + 8);
          const uint32_t hi = (d == 0.0f) ? 8u : (uint32_t)(quant_code(x[jj + 16], d, -8.0f, 7.0f) + 8);
          word |= (lo | (hi << 4)) << (8 * k);
        }
        w[i] = word;
      }
      uint4* dst = reinterpret_cast<uint4*>(p.v_qs + crow * (p.head_dim / 2) + b * 16);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      p.v_d[crow * nb + b] = dbits;
    } else {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < kBlock; ++i) a = fmaxf(a, fabsf(x[i]));
      const uint16_t dbits = f32_to_half_bits(a / 127.0f);
      const float d = half_bits_to_f32(dbits);
      uint32_t w[kBlock / 4];
#pragma unroll
      for (int i = 0; i < kBlock / 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          word |= ((uint32_t)(quant_code(x[4 * i + k], d, -127.0f, 127.0f) & 0xFF)) << (8 * k);
        w[i] = word;
      }
      uint4* dst = reinterpret_cast<uint4*>(p.v_qs + crow * p.head_dim + b * kBlock);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      p.v_d[crow * nb + b] = dbits;
    }
  }
}

int launch_append(const kvq_cache& c, const float* k_new, const float* v_new, int n_seq, int n_new,
                  const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                  hipStream_t stream) {
  AppendParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_qs = c.k_qs;
  p.k_d = c.k_d;
  p.v_qs = c.v_qs;
  p.v_d = c.v_d;
  p.seg_table = seg_table;
  p.start_pos = start_pos;
  p.n_rows = n_seq * n_new * c.n_kv_heads;
  p.n_new = n_new;
  p.n_kv_heads = c.n_kv_heads;
  p.head_dim = c.head_dim;
  p.seg_tokens = c.seg_tokens;
  p.max_segs = max_segs;
  p.v_format = c.v_format;
  const long long threads = (long long)p.n_rows * (c.head_dim / kBlock);
  const int block = 256;
  const unsigned grid = (unsigned)((threads + block - 1) / block);
  hipLaunchKernelGGL(k_append_quant, dim3(grid), dim3(block), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvq
