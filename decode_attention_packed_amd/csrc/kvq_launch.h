// Host-side launchers of the libkvq kernels.  Arguments are validated by the
// C ABI layer before any of these is called; each returns 0 or -4 (HIP error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Split plan of one attention call: the context of every (sequence, kv head)
// is cut into chunks of `chunk` tokens, one work-group each; `n_split` is the
// chunk count of the longest sequence.
struct SplitPlan {
  int chunk;
  int n_split;
};

// Byte offsets inside the caller's workspace: per-(sequence, kv head) split
// counters, then the partial outputs o and the (max, sum) pairs.
struct WorkspaceLayout {
  size_t counters;
  size_t part_o;
  size_t part_ml;
  size_t total;
};

constexpr int kTileTokens = 32;    // tokens per tile: split points fall on tile boundaries
constexpr int kChunkAlign = 256;   // one 32-token tile for each of the 8 waves of a work-group
constexpr int kMaxSplits = 64;     // splits per (sequence, kv head) the merge stages in LDS
// uint32 words from one split counter to the next: each (sequence, kv head)
// counter sits on its own 256-byte span, so that the work-groups of different
// groups finishing at the same moment do not queue on one line's atomics
constexpr int kCounterStride = 64;

SplitPlan plan_splits(const kvq_cache& c, int n_seq, int n_qtok, int n_q_heads, int max_seq_len);
WorkspaceLayout workspace_layout(const kvq_cache& c, int n_seq, int n_qtok, int n_q_heads,
                                 const SplitPlan& plan);

// k_f16: the cache's k_qs holds fp16 K rows (the fp16-K A/B cache) and k_d is unused.
int launch_append(const kvq_cache& c, const float* k_new, const float* v_new, int n_seq, int n_new,
                  const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                  hipStream_t stream, bool k_f16 = false);

bool attn_supported(int head_dim, int v_format);

// Split-K attention with the split merge fused into the last work-group;
// with n_new > 0 it first appends k_new / v_new at tokens seq_len - n_new ..
// seq_len - 1 of every sequence (in the same launch).  With dbg_isum the
// kernels also store every per-block int32 Q.K sum they form
// (kvq_debug_attn_isum); with dbg_stamps, per-work-group timestamps
// (kvq_debug_attn_timeline).
int launch_attn(const kvq_cache& c, const float* q, float* out, int n_seq, int n_qtok, int n_q_heads,
                const int32_t* seg_table, int max_segs, const int32_t* seq_len, int max_seq_len,
                const SplitPlan& plan, float sm_scale, int causal, void* workspace,
                const float* k_new, const float* v_new, int n_new, hipStream_t stream,
                int32_t* dbg_isum = nullptr, int dbg_max_len = 0,
                unsigned long long* dbg_stamps = nullptr);

// One call of a batched launch (attn_decode_packed_batch), validated.
struct AttnCall {
  const kvq_cache* cache;
  const float* q;
  float* out;
  int n_seq, n_qtok, n_q_heads;
  const int32_t* seg_table;
  int max_segs;
  const int32_t* seq_len;
  int max_seq_len;
  float sm_scale;
  int causal;
};

// All calls share head_dim, V format and layout (column or row); call i uses
// plans[i] and the workspace bytes after those of calls 0 .. i-1.
int launch_attn_batch(const AttnCall* calls, const SplitPlan* plans, int n_calls, void* workspace,
                      hipStream_t stream);

// The kernels for q4_0 V at head_dim 128 built with 12 waves per work-group
// (kvq_attn_w12.hip); launch_attn and launch_attn_batch above hand the calls
// with long enough chunks to them.
namespace w12 {
int launch_attn_batch(const AttnCall* calls, const SplitPlan* plans, int n_calls, void* workspace,
                      hipStream_t stream);
int launch_attn(const kvq_cache& c, const float* q, float* out, int n_seq, int n_qtok, int n_q_heads,
                const int32_t* seg_table, int max_segs, const int32_t* seq_len, int max_seq_len,
                const SplitPlan& plan, float sm_scale, int causal, void* workspace,
                const float* k_new, const float* v_new, int n_new, hipStream_t stream,
                int32_t* dbg_isum = nullptr, int dbg_max_len = 0,
                unsigned long long* dbg_stamps = nullptr);
}  // namespace w12

// The same attention kernels compiled for fp16 K rows (kvq_attn_f16k.hip):
// head_dim 128, column layout (query rows x 4 blocks <= 16), no append.
namespace f16k {
bool attn_supported(int head_dim, int v_format);
int launch_attn(const kvq_cache& c, const float* q, float* out, int n_seq, int n_qtok, int n_q_heads,
                const int32_t* seg_table, int max_segs, const int32_t* seq_len, int max_seq_len,
                const SplitPlan& plan, float sm_scale, int causal, void* workspace,
                const float* k_new, const float* v_new, int n_new, hipStream_t stream,
                int32_t* dbg_isum = nullptr, int dbg_max_len = 0,
                unsigned long long* dbg_stamps = nullptr);
}  // namespace f16k

int launch_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
int launch_debug_quant_q(const float* q, int n_rows, int head_dim, int8_t* codes, float* scales,
                         hipStream_t stream);
int launch_debug_isum(const kvq_cache& c, const float* q, int n_seq, int n_qtok, int n_q_heads,
                      const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                      int max_seq_len, int32_t* isum, hipStream_t stream);

}  // namespace kvq
