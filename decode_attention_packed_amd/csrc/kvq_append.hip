// kv_append_quant kernel: quantize and pack new K/V rows into the cache.
//
// Page 1 ("Flash Attention for llama.cpp on RDNA3 ... Part 1", summary and
// first body paragraph): each new K row is re-packed on the fly to int8
// codes, four per 32-bit word, with an fp16 scale per 32-block; V is written
// as q4_0 or q8_0 blocks.  32 lanes own one 32-block of one row, one element
// per lane; block maxima come from cross-lane reductions.
//
// K rows are stored token-major.  V payload and V scales are stored
// token-interleaved in tiles of 32 tokens ("BitLLM" page 3, section on what
// differs: the layout follows the reduction axis, T for S.V): inside a tile,
// byte k of the per-token row of token t sits at k * 32 + t, and scale b of
// token t at b * 32 + t.

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

struct AppendParams {
  const float* k_new;
  const float* v_new;
  uint8_t* k_qs;
  uint16_t* k_d;
  uint8_t* v_qs;
  uint16_t* v_d;
  const int32_t* seg_table;
  const int32_t* start_pos;
  int n_units;       // n_seq * n_new * n_kv_heads * head_dim / 32
  int n_new;
  int n_kv_heads;
  int head_dim;
  int seg_tokens;
  int max_segs;
  int v_format;
  int k_f16;         // 1: K rows stored as fp16 (the fp16-K A/B cache), no K scales
};

__global__ __launch_bounds__(256) void k_append_quant(AppendParams p) {
  const int nb = p.head_dim / kBlock;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int unit = gid >> 5;            // (row, block); whole half-waves share one unit
  const int e = gid & 31;               // element inside the block
  if (unit >= p.n_units) return;
  // the values first: their loads do not depend on the destination lookup
  const int row_l = unit / nb;
  const int b = unit - row_l * nb;
  const size_t src = (size_t)row_l * p.head_dim + b * kBlock + e;
  const float xk = p.k_new[src];
  const float xv = p.v_new[src];
  // a wave holds two consecutive units of one row (nb is even), so the row
  // and its destination are uniform and come from scalar loads
  const int row = __builtin_amdgcn_readfirstlane(row_l);
  const int h = row % p.n_kv_heads;
  const int j = (row / p.n_kv_heads) % p.n_new;
  const int seq = row / (p.n_kv_heads * p.n_new);

  const int pos = p.start_pos[seq] + j;
  const int segj = pos / p.seg_tokens;
  const int seg = segment_of(p.seg_table, seq, p.max_segs, segj);
  const size_t prow = ((size_t)seg * p.n_kv_heads + h) * p.seg_tokens + (pos - segj * p.seg_tokens);
  const size_t tile0 = prow & ~(size_t)(kTile - 1);   // first row of this token's 32-token tile
  const int t = (int)(prow - tile0);

  // ---- K
  if (p.k_f16) {
    reinterpret_cast<uint16_t*>(p.k_qs)[prow * p.head_dim + b * kBlock + e] = f32_to_half_bits(xk);
  } else {
    int code;
    const uint16_t dbits = quant_sym8(xk, code);
    p.k_qs[prow * p.head_dim + b * kBlock + e] = (uint8_t)code;
    if (e == 0) p.k_d[tile0 * nb + b * kTile + t] = dbits;
  }

  // ---- V
  if (p.v_format == 0) {
    uint32_t byte;
    const uint16_t dbits = quant_q4_0(xv, e, byte);
    if (e < 16) p.v_qs[tile0 * (p.head_dim / 2) + (size_t)(b * 16 + e) * kTile + t] = (uint8_t)byte;
    if (e == 0) p.v_d[tile0 * nb + b * kTile + t] = dbits;
  } else {
    int code;
    const uint16_t dbits = quant_sym8(xv, code);
    p.v_qs[tile0 * p.head_dim + (size_t)(b * kBlock + e) * kTile + t] = (uint8_t)code;
    if (e == 0) p.v_d[tile0 * nb + b * kTile + t] = dbits;
  }
}

int launch_append(const kvq_cache& c, const float* k_new, const float* v_new, int n_seq, int n_new,
                  const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                  hipStream_t stream, bool k_f16) {
  AppendParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_qs = reinterpret_cast<uint8_t*>(c.k_qs);
  p.k_d = c.k_d;
  p.v_qs = c.v_qs;
  p.v_d = c.v_d;
  p.seg_table = seg_table;
  p.start_pos = start_pos;
  p.n_units = n_seq * n_new * c.n_kv_heads * (c.head_dim / kBlock);
  p.n_new = n_new;
  p.n_kv_heads = c.n_kv_heads;
  p.head_dim = c.head_dim;
  p.seg_tokens = c.seg_tokens;
  p.max_segs = max_segs;
  p.v_format = c.v_format;
  p.k_f16 = k_f16 ? 1 : 0;
  const long long threads = (long long)p.n_units * kBlock;
  const int block = 256;
  const unsigned grid = (unsigned)((threads + block - 1) / block);
  hipLaunchKernelGGL(k_append_quant, dim3(grid), dim3(block), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvq
