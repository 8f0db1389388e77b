// Test hooks that expose the integer stages of the attention kernels: the Q
// quantization (same wave routine as the attention prologue) and the per-block
// int32 QK sums (same lane layout and dot4 chain as the split kernel).

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

__global__ __launch_bounds__(64) void k_debug_quant_q(const float* q, int head_dim, int8_t* codes,
                                                      float* scales) {
  const int row = blockIdx.x;
  quantize_q_wave(q + (size_t)row * head_dim, head_dim, codes + (size_t)row * head_dim,
                  scales + (size_t)row * (head_dim / kBlock));
}

template <int D>
__global__ __launch_bounds__(64) void k_debug_isum(const uint32_t* k_qs, const float* q,
                                                   const int32_t* seg_table, const int32_t* seq_len,
                                                   int32_t* isum, int n_kv_heads, int n_q_heads,
                                                   int n_qtok, int seg_tokens, int max_segs,
                                                   int max_seq_len) {
  constexpr int PARTS = D / 16;
  constexpr int SLOTS = 64 / PARTS;
  constexpr int NB = D / kBlock;
  __shared__ __attribute__((aligned(16))) int8_t s_qc[D];
  __shared__ float s_qd[NB];

  const int lane = threadIdx.x;
  const int part = lane % PARTS;
  const int slot = lane / PARTS;
  const int qrow = blockIdx.y;            // qtok * n_q_heads + h
  const int seq = blockIdx.z;
  const int h = qrow % n_q_heads;
  const int kvh = h / (n_q_heads / n_kv_heads);
  const size_t row = (size_t)seq * n_qtok * n_q_heads + qrow;

  quantize_q_wave(q + row * D, D, s_qc, s_qd);
  __syncthreads();
  const uint4 qv = *reinterpret_cast<const uint4*>(s_qc + 16 * part);

  const int t = blockIdx.x * SLOTS + slot;
  const int L = seq_len[seq];
  const bool valid = t < L;
  int is = 0;
  if (valid) {
    const int segj = t / seg_tokens;
    const int seg = segment_of(seg_table, seq, max_segs, segj);
    const size_t r = ((size_t)seg * n_kv_heads + kvh) * seg_tokens + (t - segj * seg_tokens);
    const uint4 kv = reinterpret_cast<const uint4*>(k_qs)[r * (D / 16) + part];
    is = dot4(qv.x, kv.x, 0);
    is = dot4(qv.y, kv.y, is);
    is = dot4(qv.z, kv.z, is);
    is = dot4(qv.w, kv.w, is);
  }
  is = isum_pair<PARTS>(is);
  if (valid && (part & 1) == 0) isum[(row * max_seq_len + t) * NB + (part >> 1)] = is;
}

int launch_debug_quant_q(const float* q, int n_rows, int head_dim, int8_t* codes, float* scales,
                         hipStream_t stream) {
  hipLaunchKernelGGL(k_debug_quant_q, dim3(n_rows), dim3(64), 0, stream, q, head_dim, codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_debug_isum(const kvq_cache& c, const float* q, int n_seq, int n_qtok, int n_q_heads,
                      const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                      int max_seq_len, int32_t* isum, hipStream_t stream) {
  const int slots = 64 / (c.head_dim / 16);
  const dim3 grid((max_seq_len + slots - 1) / slots, n_qtok * n_q_heads, n_seq);
  if (c.head_dim == 128)
    hipLaunchKernelGGL(k_debug_isum<128>, grid, dim3(64), 0, stream, c.k_qs, q, seg_table, seq_len,
                       isum, c.n_kv_heads, n_q_heads, n_qtok, c.seg_tokens, max_segs, max_seq_len);
  else
    hipLaunchKernelGGL(k_debug_isum<64>, grid, dim3(64), 0, stream, c.k_qs, q, seg_table, seq_len,
                       isum, c.n_kv_heads, n_q_heads, n_qtok, c.seg_tokens, max_segs, max_seq_len);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace kvq
