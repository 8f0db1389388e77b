// C ABI of libkvq: host-side validation, split planning and launches.
// Every check runs before the first launch, so an error return leaves device
// memory untouched.  The library never allocates; its only state is the
// static scratch array of attn_decode_packed_noalloc and, per device, that
// array's address.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "kvq.h"
#include "kvq_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// f16k: the fp16-K A/B cache (k_qs holds fp16 K rows, k_d must be NULL,
// head_dim 128 only).
int check_cache(const kvq_cache* c, bool f16k = false) {
  if (!c) return KVQ_ERR_INVALID;
  if (c->n_kv_heads < 1 || c->n_segs < 1 || c->reserved != 0) return KVQ_ERR_INVALID;
  if (c->seg_tokens < KVQ_SEG_ALIGN || c->seg_tokens % KVQ_SEG_ALIGN) return KVQ_ERR_INVALID;
  if (c->v_format != KVQ_V_Q4_0 && c->v_format != KVQ_V_Q8_0) return KVQ_ERR_INVALID;
  if (c->head_dim < KVQ_BLOCK || c->head_dim % KVQ_BLOCK) return KVQ_ERR_INVALID;
  if (c->head_dim != 128 && (f16k || c->head_dim != 64)) return KVQ_ERR_UNSUPPORTED;
  if (!c->k_qs || !c->v_qs || !c->v_d || (f16k ? c->k_d != nullptr : !c->k_d)) return KVQ_ERR_INVALID;
  if (!aligned16(c->k_qs) || (!f16k && !aligned16(c->k_d)) || !aligned16(c->v_qs) ||
      !aligned16(c->v_d))
    return KVQ_ERR_INVALID;
  return KVQ_OK;
}

// Without a segment table, sequence i uses segments i*max_segs .. i*max_segs+max_segs-1.
int check_segments(const kvq_cache* c, int n_seq, const int32_t* seg_table, int max_segs) {
  if (max_segs < 1) return KVQ_ERR_INVALID;
  if (!seg_table && (long long)n_seq * max_segs > c->n_segs) return KVQ_ERR_INVALID;
  if (seg_table && (reinterpret_cast<uintptr_t>(seg_table) & 3u)) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

int check_attn(const kvq_cache* c, const float* q, const float* out, int n_seq, int n_qtok,
               int n_q_heads, const int32_t* seg_table, int max_segs, const int32_t* seq_len,
               int max_seq_len, bool f16k = false) {
  int st = check_cache(c, f16k);
  if (st) return st;
  if (!q || !out || !seq_len || !aligned16(q) || !aligned16(out)) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(seq_len) & 3u) return KVQ_ERR_INVALID;
  if (n_seq < 1 || n_qtok < 1 || n_qtok > KVQ_MAX_QTOK || n_q_heads < 1) return KVQ_ERR_INVALID;
  if (n_q_heads % c->n_kv_heads) return KVQ_ERR_INVALID;
  if (max_seq_len < n_qtok || (long long)max_seq_len > (long long)max_segs * c->seg_tokens)
    return KVQ_ERR_INVALID;
  st = check_segments(c, n_seq, seg_table, max_segs);
  if (st) return st;
  return KVQ_OK;
}

}  // namespace

namespace kvq {

// The smallest chunk of whole tiles (at least kChunkAlign tokens) that
// covers `len` tokens in `n` splits.
static int even_chunk(long long len, long long n) {
  const long long per = (len + n - 1) / n;
  return (int)std::max<long long>(kChunkAlign, (per + kTileTokens - 1) / kTileTokens * kTileTokens);
}

SplitPlan plan_splits(const kvq_cache& c, int n_seq, int n_qtok, int n_q_heads, int max_seq_len) {
  (void)n_qtok;
  (void)n_q_heads;
  auto splits = [&](long long chunk) { return (max_seq_len + chunk - 1) / chunk; };
  int chunk = 0;
  if (const char* env = std::getenv("KVQ_CHUNK_TOKENS")) {
    chunk = std::atoi(env);
    if (chunk < kChunkAlign || chunk % kChunkAlign) chunk = 0;
  }
  if (!chunk) {
    const long long target_groups = 256;   // one work-group per CU
    const long long n_groups = (long long)n_seq * c.n_kv_heads;
    chunk = kChunkAlign;
    if (n_groups >= target_groups) {
      // Enough (sequence, kv head) groups to fill the GPU unsplit.  More,
      // shorter work-groups only add start-up latency and merges, so the
      // longest sequence splits just enough for about two groups' worth of
      // work-groups per CU: in two below 512 groups, not at all from 512
      // (ragged batch, 512 groups: 94 us unsplit, 107 us in two, 135 us in
      // 4096-token chunks).
      const long long most = std::max<long long>(1, 2 * target_groups / n_groups);
      while (chunk < (1 << 20) && splits(chunk) > most) chunk *= 2;
      chunk = even_chunk(max_seq_len, splits(chunk));
    } else if (splits(2 * kChunkAlign) == 1) {
      // Short sequences (two tiles per wave at most): one work-group per
      // group writes its rows directly, with no split merge (512 tokens, 1-4
      // kv heads: 7.9 us against 9.3 us in two splits; from 1024 tokens
      // 256-token splits are faster again).
      chunk = 2 * kChunkAlign;
    } else if (n_groups * 8 <= target_groups) {
      // Few groups (at most 32): 256 / groups splits per sequence (at most
      // kMaxSplits), each a whole number of tiles, so one work-group per CU
      // carries a near-equal share at any length.  Power-of-two chunks gave
      // 33 splits at 131073 tokens: 8 one-token work-groups in a second
      // round after the rest of the grid.
      chunk = even_chunk(max_seq_len, std::min<long long>(target_groups / n_groups, kMaxSplits));
    } else {
      // Up to 255 groups: grow the chunk while at least one work-group per CU
      // remains and the longest sequence still spreads over 8 or more.
      while (chunk < (1 << 20)) {
        const long long next = 2LL * chunk;
        if (n_groups * splits(next) < target_groups || splits(next) < 8) break;
        chunk = (int)next;
      }
      // the nearest split count, in even chunks (just past a power of two
      // the loop above leaves a near-empty last split: 9 at 131073 tokens)
      chunk = even_chunk(max_seq_len, std::max<long long>(1, (max_seq_len + chunk / 2) / chunk));
    }
  }
  // the split merge stages at most kMaxSplits partials per (sequence, kv head)
  while (splits(chunk) > kMaxSplits) chunk *= 2;
  SplitPlan p;
  p.chunk = chunk;
  p.n_split = (int)splits(chunk);
  return p;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(const kvq_cache& c, int n_seq, int n_qtok, int n_q_heads,
                                 const SplitPlan& plan) {
  const size_t rows = (size_t)n_qtok * (n_q_heads / c.n_kv_heads);
  const size_t groups = (size_t)n_seq * c.n_kv_heads;
  WorkspaceLayout w;
  w.counters = 0;
  w.part_o = round256(groups * kCounterStride * sizeof(unsigned));
  w.part_ml = w.part_o + round256(groups * plan.n_split * rows * c.head_dim * sizeof(float));
  w.total = w.part_ml + round256(groups * plan.n_split * rows * 2 * sizeof(float));
  return w;
}

}  // namespace kvq

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int kvq_cache_bytes(int n_kv_heads, int head_dim, int seg_tokens, int n_segs, int v_format,
                    size_t out_bytes[4]) {
  if (!out_bytes || n_kv_heads < 1 || n_segs < 1 || seg_tokens < 1) return KVQ_ERR_INVALID;
  if (head_dim < KVQ_BLOCK || head_dim % KVQ_BLOCK) return KVQ_ERR_INVALID;
  if (v_format != KVQ_V_Q4_0 && v_format != KVQ_V_Q8_0) return KVQ_ERR_INVALID;
  const size_t rows = (size_t)n_segs * n_kv_heads * seg_tokens;
  const size_t nb = head_dim / KVQ_BLOCK;
  out_bytes[0] = rows * head_dim;                                   // int8 K codes
  out_bytes[1] = rows * nb * 2;                                     // fp16 K scales
  out_bytes[2] = rows * (v_format == KVQ_V_Q4_0 ? head_dim / 2 : head_dim);
  out_bytes[3] = rows * nb * 2;                                     // fp16 V scales
  return KVQ_OK;
}

int kv_append_quant(const kvq_cache* cache, const float* k_new, const float* v_new, int n_seq,
                    int n_new, const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                    void* stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (!k_new || !v_new || !start_pos || !aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(start_pos) & 3u) return KVQ_ERR_INVALID;
  if (n_seq < 1 || n_new < 1) return KVQ_ERR_INVALID;
  if ((long long)n_seq * n_new * cache->n_kv_heads * cache->head_dim > 0x7fffff00LL)
    return KVQ_ERR_INVALID;
  st = check_segments(cache, n_seq, seg_table, max_segs);
  if (st) return st;
  const int r = kvq::launch_append(*cache, k_new, v_new, n_seq, n_new, seg_table, max_segs,
                                   start_pos, static_cast<hipStream_t>(stream));
  return r ? KVQ_ERR_HIP : KVQ_OK;
}

int attn_decode_packed_workspace_size(const kvq_cache* cache, int n_seq, int n_qtok, int n_q_heads,
                                      int max_seq_len, size_t* bytes) {
  int st = check_cache(cache);
  if (st) return st;
  if (!bytes || n_seq < 1 || n_qtok < 1 || n_qtok > KVQ_MAX_QTOK || n_q_heads < 1 ||
      n_q_heads % cache->n_kv_heads || max_seq_len < n_qtok)
    return KVQ_ERR_INVALID;
  if (n_qtok * (n_q_heads / cache->n_kv_heads) > KVQ_MAX_QTOK) return KVQ_ERR_UNSUPPORTED;
  const kvq::SplitPlan plan = kvq::plan_splits(*cache, n_seq, n_qtok, n_q_heads, max_seq_len);
  *bytes = kvq::workspace_layout(*cache, n_seq, n_qtok, n_q_heads, plan).total;
  return KVQ_OK;
}

namespace {

int attn_common(const kvq_cache* cache, const float* q, float* out, int n_seq, int n_qtok,
                int n_q_heads, const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                int max_seq_len, float sm_scale, int causal, void* workspace, size_t workspace_bytes,
                const float* k_new, const float* v_new, int n_new, void* stream,
                int32_t* dbg_isum = nullptr, unsigned long long* dbg_stamps = nullptr) {
  int st = check_attn(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                      max_seq_len);
  if (st) return st;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  const int group = n_q_heads / cache->n_kv_heads;
  if (n_qtok * group > KVQ_MAX_QTOK) return KVQ_ERR_UNSUPPORTED;
  if (!kvq::attn_supported(cache->head_dim, cache->v_format)) return KVQ_ERR_UNSUPPORTED;
  const kvq::SplitPlan plan = kvq::plan_splits(*cache, n_seq, n_qtok, n_q_heads, max_seq_len);
  const size_t need = kvq::workspace_layout(*cache, n_seq, n_qtok, n_q_heads, plan).total;
  if (workspace_bytes < need || !workspace) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_INVALID;
  const int r = kvq::launch_attn(*cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs,
                                 seq_len, max_seq_len, plan, sm_scale, causal ? 1 : 0, workspace,
                                 k_new, v_new, n_new, static_cast<hipStream_t>(stream), dbg_isum,
                                 max_seq_len, dbg_stamps);
  return r ? KVQ_ERR_HIP : KVQ_OK;
}

// Validate one call of a batch and convert it.
int check_call(const kvq_attn_call* a, kvq::AttnCall* out) {
  if (!a) return KVQ_ERR_INVALID;
  int st = check_attn(a->cache, a->q, a->out, a->n_seq, a->n_qtok, a->n_q_heads, a->seg_table,
                      a->max_segs, a->seq_len, a->max_seq_len);
  if (st) return st;
  if (!std::isfinite(a->sm_scale)) return KVQ_ERR_INVALID;
  if (a->n_qtok * (a->n_q_heads / a->cache->n_kv_heads) > KVQ_MAX_QTOK) return KVQ_ERR_UNSUPPORTED;
  if (!kvq::attn_supported(a->cache->head_dim, a->cache->v_format)) return KVQ_ERR_UNSUPPORTED;
  *out = {a->cache, a->q, a->out, a->n_seq, a->n_qtok, a->n_q_heads, a->seg_table, a->max_segs,
          a->seq_len, a->max_seq_len, a->sm_scale, a->causal ? 1 : 0};
  return KVQ_OK;
}

// Validate a batch; on success fills calls[], plans[] and the workspace size.
// One launch runs every call, so the split plan is joint: with fewer than
// 256 (sequence, kv head) groups in all, one chunk length for every call,
// the shortest whole number of 32-token tiles (at least 256 tokens) that
// keeps the whole grid within one work-group per CU; otherwise each call's
// own plan.
int check_batch(const kvq_attn_call* calls, int n_calls, kvq::AttnCall* out, kvq::SplitPlan* plans,
                size_t* ws_bytes) {
  if (!calls || n_calls < 1 || n_calls > KVQ_MAX_BATCH) return KVQ_ERR_INVALID;
  long long groups = 0;
  for (int i = 0; i < n_calls; ++i) {
    const int st = check_call(&calls[i], &out[i]);
    if (st) return st;
    const kvq_cache& c0 = *out[0].cache;
    const kvq_cache& c = *out[i].cache;
    if (c.head_dim != c0.head_dim || c.v_format != c0.v_format) return KVQ_ERR_UNSUPPORTED;
    const int nb = c.head_dim / KVQ_BLOCK;
    const bool rows0 = out[0].n_qtok * (out[0].n_q_heads / c0.n_kv_heads) * nb > 16;
    const bool rows = out[i].n_qtok * (out[i].n_q_heads / c.n_kv_heads) * nb > 16;
    if (rows != rows0) return KVQ_ERR_UNSUPPORTED;
    groups += (long long)out[i].n_seq * c.n_kv_heads;
  }
  if (groups >= 256) {
    for (int i = 0; i < n_calls; ++i)
      plans[i] = kvq::plan_splits(*out[i].cache, out[i].n_seq, out[i].n_qtok, out[i].n_q_heads,
                                  out[i].max_seq_len);
  } else {
    // the smallest chunk, in whole 32-token tiles, that keeps the joint grid
    // within one work-group per CU: the splits then come out nearly equal
    // (verify step: 21 splits of 6272 tokens rather than 20 of 6400 and a
    // last one of 3072)
    int chunk = kvq::kChunkAlign;
    for (;; chunk += kvq::kTileTokens) {
      long long wgs = 0;
      int most = 0;
      for (int i = 0; i < n_calls; ++i) {
        const long long sp = (out[i].max_seq_len + chunk - 1) / chunk;
        wgs += (long long)out[i].n_seq * out[i].cache->n_kv_heads * sp;
        most = (int)std::max<long long>(most, sp);
      }
      if ((wgs <= 256 && most <= kvq::kMaxSplits) || chunk >= (1 << 20)) break;
    }
    for (int i = 0; i < n_calls; ++i)
      plans[i] = {chunk, (out[i].max_seq_len + chunk - 1) / chunk};
  }
  size_t total = 0;
  for (int i = 0; i < n_calls; ++i)
    total += kvq::workspace_layout(*out[i].cache, out[i].n_seq, out[i].n_qtok, out[i].n_q_heads,
                                   plans[i]).total;
  *ws_bytes = total;
  return KVQ_OK;
}

}  // namespace

int attn_decode_packed_batch_workspace_size(const kvq_attn_call* calls, int n_calls, size_t* bytes) {
  if (!bytes) return KVQ_ERR_INVALID;
  kvq::AttnCall c[KVQ_MAX_BATCH];
  kvq::SplitPlan plans[KVQ_MAX_BATCH];
  return check_batch(calls, n_calls, c, plans, bytes);
}

int attn_decode_packed_batch(const kvq_attn_call* calls, int n_calls, void* workspace,
                             size_t workspace_bytes, void* stream) {
  kvq::AttnCall c[KVQ_MAX_BATCH];
  kvq::SplitPlan plans[KVQ_MAX_BATCH];
  size_t need = 0;
  const int st = check_batch(calls, n_calls, c, plans, &need);
  if (st) return st;
  if (workspace_bytes < need || !workspace) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_INVALID;
  return kvq::launch_attn_batch(c, plans, n_calls, workspace, static_cast<hipStream_t>(stream))
             ? KVQ_ERR_HIP
             : KVQ_OK;
}

// ---------------------------------------------------------------------------
// attn_decode_packed_noalloc: the workspace is a static device array
// ---------------------------------------------------------------------------
//
// `scratch` is this library's own device memory, one copy per GPU, held
// until the process ends.  In host code its name is only a host-side
// stand-in, so kernels and fills get the address that hipGetSymbolAddress
// reports for the current device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, or null when the
// runtime cannot report it.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Zero-fill of the split counters at the front of the scratch array (a
// kernel rather than hipMemsetAsync, so the call can be captured in a graph).
__global__ __launch_bounds__(256) void k_zero_words(unsigned* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

int attn_decode_packed_noalloc(const kvq_cache* cache, const float* q, float* out, int n_seq,
                               int n_qtok, int n_q_heads, const int32_t* seg_table, int max_segs,
                               const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                               void* stream) {
  int st = check_attn(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                      max_seq_len);
  if (st) return st;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  if (n_qtok * (n_q_heads / cache->n_kv_heads) > KVQ_MAX_QTOK) return KVQ_ERR_UNSUPPORTED;
  if (!kvq::attn_supported(cache->head_dim, cache->v_format)) return KVQ_ERR_UNSUPPORTED;
  const kvq::SplitPlan plan = kvq::plan_splits(*cache, n_seq, n_qtok, n_q_heads, max_seq_len);
  const kvq::WorkspaceLayout ws = kvq::workspace_layout(*cache, n_seq, n_qtok, n_q_heads, plan);
  if (ws.total > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  void* base = scratch_ptr();
  if (!base) return KVQ_ERR_HIP;
  // the array keeps the previous call's bytes: its counters must start at zero
  const int words = (int)(ws.part_o / sizeof(unsigned));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_zero_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                     static_cast<unsigned*>(base), words);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  const int r = kvq::launch_attn(*cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs,
                                 seq_len, max_seq_len, plan, sm_scale, causal ? 1 : 0, base, nullptr,
                                 nullptr, 0, s);
  return r ? KVQ_ERR_HIP : KVQ_OK;
}

int attn_decode_packed(const kvq_cache* cache, const float* q, float* out, int n_seq, int n_qtok,
                       int n_q_heads, const int32_t* seg_table, int max_segs,
                       const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return attn_common(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                     max_seq_len, sm_scale, causal, workspace, workspace_bytes, nullptr, nullptr, 0,
                     stream);
}

int attn_decode_packed_append(const kvq_cache* cache, const float* q, const float* k_new,
                              const float* v_new, float* out, int n_seq, int n_qtok, int n_q_heads,
                              int n_new, const int32_t* seg_table, int max_segs,
                              const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_INVALID;
  if (n_new < 1 || n_new > KVQ_MAX_APPEND || n_new > max_seq_len) return KVQ_ERR_INVALID;
  if (cache && n_seq > 0 &&
      (long long)n_seq * n_new * cache->n_kv_heads * cache->head_dim > 0x7fffff00LL)
    return KVQ_ERR_INVALID;
  return attn_common(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                     max_seq_len, sm_scale, causal, workspace, workspace_bytes, k_new, v_new, n_new,
                     stream);
}

int kvq_f16k_cache_bytes(int n_kv_heads, int head_dim, int seg_tokens, int n_segs, int v_format,
                         size_t out_bytes[4]) {
  const int st = kvq_cache_bytes(n_kv_heads, head_dim, seg_tokens, n_segs, v_format, out_bytes);
  if (st) return st;
  out_bytes[0] *= 2;   // fp16 K rows
  out_bytes[1] = 0;    // no K scales
  return KVQ_OK;
}

int kv_append_f16k(const kvq_cache* cache, const float* k_new, const float* v_new, int n_seq,
                   int n_new, const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                   void* stream) {
  int st = check_cache(cache, true);
  if (st) return st;
  if (!k_new || !v_new || !start_pos || !aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(start_pos) & 3u) return KVQ_ERR_INVALID;
  if (n_seq < 1 || n_new < 1) return KVQ_ERR_INVALID;
  if ((long long)n_seq * n_new * cache->n_kv_heads * cache->head_dim > 0x7fffff00LL)
    return KVQ_ERR_INVALID;
  st = check_segments(cache, n_seq, seg_table, max_segs);
  if (st) return st;
  const int r = kvq::launch_append(*cache, k_new, v_new, n_seq, n_new, seg_table, max_segs,
                                   start_pos, static_cast<hipStream_t>(stream), true);
  return r ? KVQ_ERR_HIP : KVQ_OK;
}

int attn_decode_f16k_workspace_size(const kvq_cache* cache, int n_seq, int n_qtok, int n_q_heads,
                                    int max_seq_len, size_t* bytes) {
  if (!bytes) return KVQ_ERR_INVALID;
  int st = check_cache(cache, true);
  if (st) return st;
  if (n_seq < 1 || n_qtok < 1 || n_q_heads < 1 || n_q_heads % cache->n_kv_heads || max_seq_len < 1)
    return KVQ_ERR_INVALID;
  const kvq::SplitPlan plan = kvq::plan_splits(*cache, n_seq, n_qtok, n_q_heads, max_seq_len);
  *bytes = kvq::workspace_layout(*cache, n_seq, n_qtok, n_q_heads, plan).total;
  return KVQ_OK;
}

int attn_decode_f16k(const kvq_cache* cache, const float* q, float* out, int n_seq, int n_qtok,
                     int n_q_heads, const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                     int max_seq_len, float sm_scale, int causal, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_attn(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                      max_seq_len, true);
  if (st) return st;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  // column layout only: query rows of a kv group times 4 blocks fill at most 16 MFMA columns
  if (n_qtok * (n_q_heads / cache->n_kv_heads) * (cache->head_dim / KVQ_BLOCK) > 16)
    return KVQ_ERR_UNSUPPORTED;
  if (!kvq::f16k::attn_supported(cache->head_dim, cache->v_format)) return KVQ_ERR_UNSUPPORTED;
  const kvq::SplitPlan plan = kvq::plan_splits(*cache, n_seq, n_qtok, n_q_heads, max_seq_len);
  const size_t need = kvq::workspace_layout(*cache, n_seq, n_qtok, n_q_heads, plan).total;
  if (workspace_bytes < need || !workspace) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_INVALID;
  const int r = kvq::f16k::launch_attn(*cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs,
                                       seq_len, max_seq_len, plan, sm_scale, causal ? 1 : 0,
                                       workspace, nullptr, nullptr, 0,
                                       static_cast<hipStream_t>(stream));
  return r ? KVQ_ERR_HIP : KVQ_OK;
}

int kvq_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || !aligned16(buf) || bytes % 16 || bytes == 0) return KVQ_ERR_INVALID;
  return kvq::launch_debug_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream))
             ? KVQ_ERR_HIP
             : KVQ_OK;
}

int kvq_debug_quant_q(const float* q, int n_rows, int head_dim, int8_t* codes, float* scales,
                      void* stream) {
  if (!q || !codes || !scales || !aligned16(q) || !aligned16(codes) || !aligned16(scales))
    return KVQ_ERR_INVALID;
  if (n_rows < 1) return KVQ_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  return kvq::launch_debug_quant_q(q, n_rows, head_dim, codes, scales,
                                   static_cast<hipStream_t>(stream))
             ? KVQ_ERR_HIP
             : KVQ_OK;
}

int kvq_debug_attn_isum(const kvq_cache* cache, const float* q, float* out, int n_seq, int n_qtok,
                        int n_q_heads, const int32_t* seg_table, int max_segs,
                        const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                        void* workspace, size_t workspace_bytes, int32_t* isum, void* stream) {
  if (!isum || !aligned16(isum)) return KVQ_ERR_INVALID;
  return attn_common(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                     max_seq_len, sm_scale, causal, workspace, workspace_bytes, nullptr, nullptr, 0,
                     stream, isum);
}

int kvq_debug_attn_timeline(const kvq_cache* cache, const float* q, float* out, int n_seq,
                            int n_qtok, int n_q_heads, const int32_t* seg_table, int max_segs,
                            const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                            void* workspace, size_t workspace_bytes, uint64_t* stamps,
                            void* stream) {
  if (!stamps || !aligned16(stamps)) return KVQ_ERR_INVALID;
  return attn_common(cache, q, out, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                     max_seq_len, sm_scale, causal, workspace, workspace_bytes, nullptr, nullptr, 0,
                     stream, nullptr, reinterpret_cast<unsigned long long*>(stamps));
}

int kvq_debug_qk_isum(const kvq_cache* cache, const float* q, int n_seq, int n_qtok, int n_q_heads,
                      const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                      int max_seq_len, int32_t* isum, void* stream) {
  int st = check_attn(cache, q, q, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                      max_seq_len);
  if (st) return st;
  if (!isum || !aligned16(isum)) return KVQ_ERR_INVALID;
  if (n_qtok * (n_q_heads / cache->n_kv_heads) > KVQ_MAX_QTOK) return KVQ_ERR_UNSUPPORTED;
  return kvq::launch_debug_isum(*cache, q, n_seq, n_qtok, n_q_heads, seg_table, max_segs, seq_len,
                                max_seq_len, isum, static_cast<hipStream_t>(stream))
             ? KVQ_ERR_HIP
             : KVQ_OK;
}

}  // extern "C"
