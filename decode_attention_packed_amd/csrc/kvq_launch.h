// Host-side launchers of the libkvq kernels.  Arguments are validated by the
// C ABI layer before any of these is called; each returns 0 or -4 (HIP error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Split plan of one attention call: the context of every (sequence, kv head)
// is cut into `n_split` chunks of `chunk` tokens.
struct SplitPlan {
  int chunk;
  int n_split;
};

SplitPlan plan_splits(const kvq_cache& c, int n_seq, int n_qtok, int n_q_heads, int max_seq_len);
size_t workspace_bytes(const kvq_cache& c, int n_seq, int n_qtok, int n_q_heads,
                       const SplitPlan& plan);

int launch_append(const kvq_cache& c, const float* k_new, const float* v_new, int n_seq, int n_new,
                  const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                  hipStream_t stream);

// Single-query split kernel (n_qtok == 1) followed by the split combine.
int launch_attn_sq(const kvq_cache& c, const float* q, float* out, int n_seq, int n_q_heads,
                   const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                   const SplitPlan& plan, float sm_scale, void* workspace, hipStream_t stream);

// Combine per-split partials (m, l, o) into the output rows.
int launch_combine(const float* part_o, const float* part_ml, float* out, int n_rows, int n_split,
                   int head_dim, hipStream_t stream);

bool attn_sq_supported(int head_dim, int group, int v_format);

int launch_debug_quant_q(const float* q, int n_rows, int head_dim, int8_t* codes, float* scales,
                         hipStream_t stream);
int launch_debug_isum(const kvq_cache& c, const float* q, int n_seq, int n_qtok, int n_q_heads,
                      const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                      int max_seq_len, int32_t* isum, hipStream_t stream);

}  // namespace kvq
