// Test hooks that expose the integer stages of the attention kernel: the Q
// quantization (same wave routine as the attention prologue) and the per-block
// int32 QK sums (same Q prologue, operand layout and int8 MFMA as the split
// kernel).

#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_qk.h"

namespace kvq {

__global__ __launch_bounds__(64) void k_debug_quant_q(const float* q, int head_dim, int8_t* codes,
                                                      float* scales) {
  const int row = blockIdx.x;
  quantize_q_wave(q + (size_t)row * head_dim, head_dim, codes + (size_t)row * head_dim,
                  scales + (size_t)row * (head_dim / kBlock));
}

// One wave per (16 tokens, kv head, sequence): isum[seq][j][h][t][b] for every
// query row (j, h) of the kv group and every block b.
template <int D>
__global__ __launch_bounds__(64) void k_debug_isum(const uint32_t* k_qs, const float* q,
                                                   const int32_t* seg_table, const int32_t* seq_len,
                                                   int32_t* isum, int n_kv_heads, int n_q_heads,
                                                   int n_qtok, int seg_tokens, int max_segs,
                                                   int max_seq_len) {
  constexpr int NB = D / kBlock;
  __shared__ __attribute__((aligned(16))) int8_t s_qc[kRows * D];
  __shared__ float s_qd[kRows * NB];
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int kvh = blockIdx.y, seq = blockIdx.z;
  const int G = n_q_heads / n_kv_heads;
  const int R = n_qtok * G;
  quantize_group_rows<D>(q, seq, n_qtok, n_q_heads, kvh, G, R, 0, 1, s_qc, s_qd);
  __syncthreads();
  long qa[NB];
  load_q_operands<D>(s_qc, qa);

  const int t = blockIdx.x * 16 + col;
  const int L = seq_len[seq];
  long kb[NB];
  for (int b = 0; b < NB; ++b) kb[b] = 0;
  if (t < L) {
    const int segj = t / seg_tokens;
    const int seg = segment_of(seg_table, seq, max_segs, segj);
    const size_t r = ((size_t)seg * n_kv_heads + kvh) * seg_tokens + (t - segj * seg_tokens);
    load_k_operands<D>(reinterpret_cast<const uint8_t*>(k_qs) + r * D, kb);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const v4i c = qk_block_mfma(qa[b], kb[b]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * grp + i;
      if (row < R && t < L) {
        const int j = row / G, h = kvh * G + row % G;
        isum[((((size_t)seq * n_qtok + j) * n_q_heads + h) * max_seq_len + t) * NB + b] = c[i];
      }
    }
  }
}

// Plain streaming read of a buffer with 16-byte nontemporal loads, eight per
// thread in flight: the HBM read ceiling the attention kernels are measured
// against (they read the K/V stream with the same hint).  Each work-group
// reads one contiguous span; the xor of the data is stored only in the
// unlikely case that it equals a sentinel, so the loads cannot be dropped.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_debug_stream_read(const v4u* src, size_t n16,
                                                           uint32_t* sink) {
  constexpr int U = 8;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = per * blockIdx.x;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  size_t base = b0;
  for (; base + (size_t)256 * U <= b1; base += (size_t)256 * U) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + base + u * 256 + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (size_t i = base + threadIdx.x; i < b1; i += 256) {
    const v4u x = __builtin_nontemporal_load(src + i);
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

int launch_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_debug_stream_read, dim3(1024), dim3(256), 0, stream,
                     static_cast<const v4u*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_debug_quant_q(const float* q, int n_rows, int head_dim, int8_t* codes, float* scales,
                         hipStream_t stream) {
  hipLaunchKernelGGL(k_debug_quant_q, dim3(n_rows), dim3(64), 0, stream, q, head_dim, codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_debug_isum(const kvq_cache& c, const float* q, int n_seq, int n_qtok, int n_q_heads,
                      const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                      int max_seq_len, int32_t* isum, hipStream_t stream) {
  const dim3 grid((max_seq_len + 15) / 16, c.n_kv_heads, n_seq);
  if (c.head_dim == 128)
    hipLaunchKernelGGL(k_debug_isum<128>, grid, dim3(64), 0, stream, c.k_qs, q, seg_table, seq_len,
                       isum, c.n_kv_heads, n_q_heads, n_qtok, c.seg_tokens, max_segs, max_seq_len);
  else
    hipLaunchKernelGGL(k_debug_isum<64>, grid, dim3(64), 0, stream, c.k_qs, q, seg_table, seq_len,
                       isum, c.n_kv_heads, n_q_heads, n_qtok, c.seg_tokens, max_segs, max_seq_len);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvq
