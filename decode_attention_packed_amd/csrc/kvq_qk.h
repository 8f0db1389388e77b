// QK^T pieces shared by the attention kernel and its integer test hook:
// the per-group Q quantization prologue and the per-block int8 MFMA.
//
// MFMA operand layout (v_mfma_*_16x16x32_*, wave64): lane l supplies row or
// column c = l % 16 and the 8 contraction elements of group g = l / 16; the
// 16x16 result sits in 4 registers per lane, register i holding row
// 4*g + i of column c.  Q and K fill the contraction slots of one 32-block
// the same way (group g, slot j <-> element 32b + 8g + j), so every block
// gives its own int32 dot sums, as the per-block scales require.
#pragma once

#include "kvq_device.h"

namespace kvq {

// Quantize the query rows of one kv group into LDS.  Row r < rows is query
// token r / group, head kv_head * group + r % group; rows >= rows are zero.
// Called by every wave of the work-group (waves take rows round-robin); the
// caller synchronizes afterwards.
template <int D>
__device__ __forceinline__ void quantize_group_rows(const float* q, int seq, int n_qtok,
                                                    int n_q_heads, int kv_head, int group, int rows,
                                                    int wave, int n_waves, int8_t* s_qc,
                                                    float* s_qd) {
  constexpr int NB = D / kBlock;
  const int lane = __lane_id();
  for (int r = wave; r < kRows; r += n_waves) {
    if (r < rows) {
      const int j = r / group;
      const int h = kv_head * group + r % group;
      quantize_q_wave(q + (((size_t)seq * n_qtok + j) * n_q_heads + h) * D, D, s_qc + r * D,
                      s_qd + r * NB);
    } else {
      for (int e = lane; e < D; e += 64) s_qc[r * D + e] = 0;
      if (lane < NB) s_qd[r * NB + lane] = 0.0f;
    }
  }
}

// A operands of the QK MFMA for this lane: Q codes of row l % 16, elements
// 32b + 8(l/16) .. +8 of every block b.
template <int D>
__device__ __forceinline__ void load_q_operands(const int8_t* s_qc, long (&qa)[D / kBlock]) {
  const int lane = __lane_id();
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int b = 0; b < D / kBlock; ++b)
    qa[b] = *reinterpret_cast<const long*>(s_qc + c * D + kBlock * b + 8 * g);
}

// K codes of one token row for this lane (same element slots as the Q operand).
template <int D>
__device__ __forceinline__ void load_k_operands(const uint8_t* krow, long (&kb)[D / kBlock]) {
  const int g = __lane_id() >> 4;
#pragma unroll
  for (int b = 0; b < D / kBlock; ++b)
    kb[b] = *reinterpret_cast<const long*>(krow + kBlock * b + 8 * g);
}

__device__ __forceinline__ v4i qk_block_mfma(long qa, long kb) {
  const v4i zero = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(qa, kb, zero, 0, 0, 0);
}

}  // namespace kvq
