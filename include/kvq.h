/*
 * kvq.h - C ABI of libkvq: decode attention over a packed, quantized KV cache
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation comes from "Flash Attention for llama.cpp on RDNA3 ...
 * Part 1" (page 1): K is stored as an 8-bit payload packed four values to a
 * 32-bit word plus an fp16 scale, re-packed as tokens arrive, and QK^T runs as
 * packed int8 dot products; V is kept as q4_0 or q8_0 blocks (body text and
 * the two KLD tables).  The 47% K saving in that page's title fixes the block
 * at 32 elements with one fp16 scale.  Append-only segments follow "BitLLM"
 * (page 3), section "how it differs"; nibble placement follows its section
 * "how to use" (two aligned 4-bit values per byte).
 *
 * Conventions for every entry point:
 *  - Return KVQ_OK (0) or a negative kvq_status.  All arguments are checked on
 *    the host before anything is launched, so an error return has no side
 *    effects on device memory.
 *  - Pointers named "device" point to GPU memory owned by the caller; the
 *    library never allocates, frees, synchronizes or prints.  Its only state
 *    is the static scratch array of attn_decode_packed_noalloc and that
 *    array's address per device.  Device pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; device faults surface at the caller's next sync.
 *  - Contents of device index arrays (segment tables, lengths, positions) are
 *    preconditions and are not checked.  Inputs must be finite.
 *  - Calls are reentrant; concurrent calls that write the same cache rows or
 *    the same workspace race.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1
#define KVQ_BLOCK 32            /* elements per quantization block along head_dim */
#define KVQ_SEG_ALIGN 64        /* seg_tokens must be a positive multiple of this */
#define KVQ_MAX_QTOK 16         /* query tokens x query heads per kv head, at most */
#define KVQ_MAX_APPEND 16       /* tokens one fused append-and-attend call appends per sequence */
#define KVQ_MAX_BATCH 4         /* calls one attn_decode_packed_batch launch runs */

enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,      /* bad pointer, alignment, shape or value */
  KVQ_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim, group size, format */
  KVQ_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  KVQ_ERR_HIP = -4           /* the HIP runtime reported a launch error */
};

enum kvq_v_format {
  KVQ_V_Q4_0 = 0,  /* 32-block: fp16 d, 16 bytes; value = d * (nibble - 8) */
  KVQ_V_Q8_0 = 1   /* 32-block: fp16 d, 32 int8 codes; value = d * code */
};

/*
 * A packed KV cache.  All four planes are device memory owned by the caller,
 * laid out [n_segs][n_kv_heads][seg_tokens][...]:
 *   k_qs  uint32 [..][head_dim/4]   int8 K codes of one token per row,
 *                                   byte k of word w = element 4w+k
 *   k_d   uint16 [..][head_dim/32]  fp16 bit patterns, one per 32-block (tiled, below)
 *   v_qs  uint8  [..][vrow]         V payload, vrow = head_dim/2 (q4_0) or head_dim (q8_0)
 *   v_d   uint16 [..][head_dim/32]  fp16 bit patterns (tiled, below)
 * K codes are token-major.  The scale planes and the V payload are
 * token-interleaved in tiles of 32 tokens (rows 32i .. 32i+31 of a segment):
 * inside a tile, scale b of token t sits at scale slot b*32 + t (K and V alike)
 * and byte k of token t's q4_0/q8_0 row at byte k*32 + t, so the token axis,
 * the reduction axis of P.V, is contiguous ("BitLLM", page 3, on matching the
 * layout to the reduction axis).  A q4_0 row holds, per 32-block, bytes
 * j = 0..15 = nibble(element j) | nibble(element j+16) << 4.
 * Token t of sequence i lives in segment seg_table[i*max_segs + t/seg_tokens]
 * (or segment i*max_segs + t/seg_tokens when no table is given), at row
 * t % seg_tokens.  A contiguous cache is one segment per sequence.
 * K codes: a = max|x|, d = fp16(a/127), c = clamp(rne(x/d), -127, 127).
 * q4_0:    m = first element of largest |x|, d = fp16(m/-8),
 *          n = clamp(rne(x/d) + 8, 0, 15).   q8_0 is the K rule.
 */
typedef struct kvq_cache {
  int32_t n_kv_heads;   /* >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t seg_tokens;   /* tokens per segment, multiple of KVQ_SEG_ALIGN */
  int32_t n_segs;       /* segments in each plane */
  int32_t v_format;     /* enum kvq_v_format */
  int32_t reserved;     /* must be 0 */
  uint32_t* k_qs;       /* device */
  uint16_t* k_d;        /* device */
  uint8_t* v_qs;        /* device */
  uint16_t* v_d;        /* device */
} kvq_cache;

/* ABI version of the loaded library (KVQ_ABI_VERSION). */
int kvq_abi_version(void);

/* Static text for a status code; never NULL. */
const char* kvq_status_string(int status);

/*
 * Bytes of each plane (k_qs, k_d, v_qs, v_d) for a cache of the given shape,
 * written to out_bytes[0..3] (host array).  Host only.  Per token and kv head
 * K takes head_dim + 2*head_dim/32 bytes, i.e. 34 bytes per 32 elements, which
 * is the 47% saving over fp16 K given in page 1's title (1 - 34/64).
 */
int kvq_cache_bytes(int n_kv_heads, int head_dim, int seg_tokens, int n_segs,
                    int v_format, size_t out_bytes[4]);

/*
 * kv_append_quant: quantize and pack new K/V rows into the cache (page 1:
 * the K payload is re-packed as it is written; V is written as q4_0/q8_0).
 *   k_new, v_new  device float [n_seq][n_new][n_kv_heads][head_dim]; n_seq
 *                 and n_new at least 1 (KVQ_ERR_INVALID otherwise)
 *   start_pos     device int32 [n_seq]; row j of sequence i goes to token
 *                 start_pos[i] + j, which must be < max_segs*seg_tokens and
 *                 must map to a segment < n_segs
 *   seg_table     device int32 [n_seq][max_segs] or NULL (see kvq_cache)
 * Output bits are a pure function of the inputs (bit-exact, deterministic).
 * Rows of different calls or sequences must not target the same token.
 */
int kv_append_quant(const kvq_cache* cache, const float* k_new, const float* v_new,
                    int n_seq, int n_new, const int32_t* seg_table, int max_segs,
                    const int32_t* start_pos, void* stream);

/*
 * Workspace bytes attn_decode_packed needs for this shape (host only).  The
 * workspace is caller-owned device memory holding per-split softmax partials
 * and one split counter per (sequence, kv head), each on its own 256 bytes
 * at the front.  It must be zero-filled
 * before its first use; every completed call leaves the counters at zero, so
 * it can be reused by later calls on the same stream without clearing.
 * Calls that overlap in time must use different workspaces.
 */
int attn_decode_packed_workspace_size(const kvq_cache* cache, int n_seq, int n_qtok,
                                      int n_q_heads, int max_seq_len, size_t* bytes);

/*
 * attn_decode_packed: one decode step of attention over the packed cache
 * (page 1, "Flash Attention for llama.cpp on RDNA3 ... Part 1": summary and
 * first body paragraph -- the kernel reads the 8-bit K payload, four values
 * per 32-bit word, with its fp16 scale and feeds it straight into an integer
 * dot product, with no fp16 K buffer; body and KLD tables -- V as q4_0 or
 * q8_0; the title's flash attention -- an online softmax over the context).
 *   q        device float [n_seq][n_qtok][n_q_heads][head_dim]
 *   out      device float [n_seq][n_qtok][n_q_heads][head_dim]
 *   seq_len  device int32 [n_seq], each in [max(1, n_qtok), max_seq_len]
 *   max_seq_len  host bound on seq_len (sizes the split grid)
 *   n_seq, n_qtok (at most KVQ_MAX_QTOK), n_q_heads and max_seq_len must be
 *   at least 1: an empty call is KVQ_ERR_INVALID, not a no-op
 *   sm_scale softmax scale (1/sqrt(head_dim) in the usual model)
 *   causal   if nonzero, query j sits at position seq_len - n_qtok + j and
 *            sees tokens up to and including that position; otherwise every
 *            query sees all seq_len tokens
 * Query head h reads kv head h / (n_q_heads / n_kv_heads).  Q is quantized to
 * int8 per 32-block with an fp32 scale (a = max|q|, d = a/127, codes as for K),
 * QK^T is summed in int32 per block and rescaled in fp32, softmax runs per
 * context split with an online maximum, V is dequantized inside the
 * weighted sum (each weight p times the V block scale rounded once to fp16,
 * the sum kept in fp32), and the splits are merged by the last work-group of
 * each (sequence, kv head), or, for more than 4 query rows per kv head at
 * head_dim 128 (8 at 64), by a second launch on the same stream.
 * n_qtok * (n_q_heads / n_kv_heads) must be at most 16 (KVQ_ERR_UNSUPPORTED
 * otherwise).  The weights enter P.V as fp16 values 2^s * p * d_v (s = 4 for
 * q4_0, 8 for q8_0, cancelled by the normalization), which keeps small V
 * accurate (relative error at V scaled by 1e-3 as at unit scale) and
 * requires every cached V block's largest magnitude to be below 32000;
 * larger values overflow the fp16 operand (undefined output).
 * The split plan depends only on the shape arguments (n_seq, n_qtok,
 * n_q_heads, max_seq_len and the cache geometry; the environment variable
 * KVQ_CHUNK_TOKENS, a multiple of 256, overrides its split size for tests);
 * for a given plan the output bits are a pure function of the inputs,
 * identical from call to call.
 */
int attn_decode_packed(const kvq_cache* cache, const float* q, float* out, int n_seq,
                       int n_qtok, int n_q_heads, const int32_t* seg_table, int max_segs,
                       const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_packed_noalloc: attn_decode_packed for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes no workspace: the split
 * partials and counters live in a static device array of this library,
 * KVQ_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The call
 * allocates and frees nothing; it enqueues a small fill kernel that zeroes
 * the counters, then the attention kernels, on `stream`.
 *   Arguments, layout, output and errors are those of attn_decode_packed,
 *   except: KVQ_ERR_WORKSPACE when the call's workspace
 *   (attn_decode_packed_workspace_size) exceeds KVQ_NOALLOC_SCRATCH_BYTES,
 *   before anything is launched; KVQ_ERR_HIP when the array's device address
 *   cannot be obtained.  The output equals attn_decode_packed's bit for bit
 *   (same kernels, same split plan).
 *   The device current on the calling thread must be the one `stream` and
 *   the buffers belong to; its copy of the array is looked up on that
 *   device's first call and kept.
 *   Every call on one GPU shares that GPU's array: calls that may overlap in
 *   time on one GPU (different streams, or threads) race and give undefined
 *   results; calls in order on one stream are safe.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)
int attn_decode_packed_noalloc(const kvq_cache* cache, const float* q, float* out, int n_seq,
                               int n_qtok, int n_q_heads, const int32_t* seg_table, int max_segs,
                               const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                               void* stream);

/*
 * attn_decode_packed_append: one decode step that first appends new rows and
 * then attends, in a single launch.  The result (cache contents and output)
 * is that of kv_append_quant with start_pos[i] = seq_len[i] - n_new followed
 * by attn_decode_packed with the same arguments: page 1 re-packs each new
 * K row as it is written and attends over the packed cache, and the decode
 * step appends the token it attends from.
 *   k_new, v_new  device float [n_seq][n_new][n_kv_heads][head_dim], written
 *                 at tokens seq_len[i] - n_new .. seq_len[i] - 1
 *   n_new         1 .. KVQ_MAX_APPEND, and n_new <= seq_len[i] for every i
 *                 (n_new = n_qtok with causal set is the verify step: the
 *                 draft tokens are appended and each query sees the tokens
 *                 up to its own)
 * All other arguments, the workspace and the errors are those of
 * attn_decode_packed.  The appended rows are written once the work-group
 * that holds them has read its part of the cache, so they need not be in
 * the cache beforehand.
 *
 * Speculative accept / rollback: after a verify step that appended n draft
 * rows, accepting k of them needs no call and moves no data.  The caller's
 * length becomes seq_len[i] - n + k; rows past it are never read, and the
 * next call appends over them.  The same holds for a plain rewind of a
 * sequence to any shorter length.
 */
int attn_decode_packed_append(const kvq_cache* cache, const float* q, const float* k_new,
                              const float* v_new, float* out, int n_seq, int n_qtok,
                              int n_q_heads, int n_new, const int32_t* seg_table, int max_segs,
                              const int32_t* seq_len, int max_seq_len, float sm_scale,
                              int causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hooks: expose the integer stages of the hot path so they can be
 * compared bit for bit with a reference.
 * kvq_debug_quant_q: Q quantization exactly as the attention kernels do it.
 *   q       device float [n_rows][head_dim]
 *   codes   device int8  [n_rows][head_dim]
 *   scales  device float [n_rows][head_dim/32]
 * kvq_debug_qk_isum: per-block int32 sums of Q codes times K codes.
 *   isum    device int32 [n_seq][n_qtok][n_q_heads][max_seq_len][head_dim/32];
 *           entries for tokens >= seq_len[i] are left untouched.
 */
int kvq_debug_quant_q(const float* q, int n_rows, int head_dim, int8_t* codes, float* scales,
                      void* stream);
/*
 * attn_decode_packed_batch: several attn_decode_packed calls in one launch.
 * Page 1's speculative-verify step attends over two caches per step (the
 * main model's and the draft's); one launch lets the two overlap their fixed
 * latencies (start-up, split merge) instead of paying them in turn.
 *   calls    n_calls (1 .. KVQ_MAX_BATCH) call descriptions, each with the
 *            meaning, layout and checks of attn_decode_packed's arguments
 *            (host memory; read during the call only)
 * Every call's cache must have the same head_dim and V format, and every
 * call the same MFMA layout (query rows x 32-blocks <= 16 for all calls, or
 * > 16 for all), else KVQ_ERR_UNSUPPORTED.  The workspace holds each call's
 * workspace in turn (attn_decode_packed_batch_workspace_size); the split
 * plan is made for the whole launch, so the bytes differ from the separate
 * calls'.  The result of each call is that of attn_decode_packed up to
 * rounding (the split points may differ).  Errors before any launch.
 */
typedef struct kvq_attn_call {
  const kvq_cache* cache;
  const float* q;
  float* out;
  int32_t n_seq;
  int32_t n_qtok;
  int32_t n_q_heads;
  const int32_t* seg_table;
  int32_t max_segs;
  const int32_t* seq_len;
  int32_t max_seq_len;
  float sm_scale;
  int32_t causal;
} kvq_attn_call;

int attn_decode_packed_batch_workspace_size(const kvq_attn_call* calls, int n_calls, size_t* bytes);
int attn_decode_packed_batch(const kvq_attn_call* calls, int n_calls, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * fp16-K reference for A/B measurements (not the method).  Page 1 compares
 * its packed int8 K with K kept as fp16; these calls run the same attention
 * kernels on a cache whose K is plain fp16 rows, so both can be timed on the
 * same hardware and the time compared with the bytes each moves.
 *
 * The cache is a kvq_cache with head_dim 128 whose k_qs points to binary16 K
 * rows [seg][kv_head][token][128] (256 bytes per token) and whose k_d is
 * NULL; V is stored exactly as in the packed cache.  kvq_f16k_cache_bytes
 * gives the plane sizes (out_bytes[1] = 0).  kv_append_f16k writes K as
 * fp16 (round to nearest even) and V as kv_append_quant does.
 * attn_decode_f16k computes softmax(sm_scale * q16 . k16) v over the cache,
 * with q16 = q rounded to binary16 and the dot in fp32; it takes the column
 * layout's shapes only (n_qtok * n_q_heads / n_kv_heads <= 4, else
 * KVQ_ERR_UNSUPPORTED) and no appended rows.  Arguments, workspace and
 * errors otherwise as attn_decode_packed.
 */
int kvq_f16k_cache_bytes(int n_kv_heads, int head_dim, int seg_tokens, int n_segs, int v_format,
                         size_t out_bytes[4]);
int kv_append_f16k(const kvq_cache* cache, const float* k_new, const float* v_new, int n_seq,
                   int n_new, const int32_t* seg_table, int max_segs, const int32_t* start_pos,
                   void* stream);
int attn_decode_f16k_workspace_size(const kvq_cache* cache, int n_seq, int n_qtok, int n_q_heads,
                                    int max_seq_len, size_t* bytes);
int attn_decode_f16k(const kvq_cache* cache, const float* q, float* out, int n_seq, int n_qtok,
                     int n_q_heads, const int32_t* seg_table, int max_segs, const int32_t* seq_len,
                     int max_seq_len, float sm_scale, int causal, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * kvq_debug_stream_read: measurement hook, not part of the method.  Reads
 * `bytes` (a nonzero multiple of 16) of device memory at `buf` (16-byte
 * aligned) with plain 16-byte loads and discards them; `sink` (device, one
 * uint32) is written only by chance.  Timed, it gives the HBM read rate a
 * streaming kernel reaches on the device, the ceiling for the kernels above.
 */
int kvq_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int kvq_debug_qk_isum(const kvq_cache* cache, const float* q, int n_seq, int n_qtok,
                      int n_q_heads, const int32_t* seg_table, int max_segs,
                      const int32_t* seq_len, int max_seq_len, int32_t* isum, void* stream);

/*
 * kvq_debug_attn_isum: test hook.  Runs attn_decode_packed (same arguments,
 * workspace, split plan, kernel build and output) with kernels that also
 * store every per-block int32 sum of Q codes times K codes that their tiles
 * form, as the matrix cores produce it from the K rows in LDS:
 *   isum    device int32 [n_seq][n_qtok][n_q_heads][max_seq_len][head_dim/32]
 *           (16-byte aligned); entry [i][j][h][t][b] is written for every
 *           token t < seq_len[i], every block b and every query head h, and
 *           is left untouched otherwise.
 * Page 1 (summary, body): 8-bit K values go four to a word straight into the
 * integer dot, so these sums are exact integers that a reference must match
 * bit for bit.  Errors as attn_decode_packed; KVQ_ERR_INVALID for a NULL or
 * misaligned isum.
 */
int kvq_debug_attn_isum(const kvq_cache* cache, const float* q, float* out, int n_seq, int n_qtok,
                        int n_q_heads, const int32_t* seg_table, int max_segs,
                        const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                        void* workspace, size_t workspace_bytes, int32_t* isum, void* stream);

/*
 * kvq_debug_attn_timeline: measurement hook, not part of the method.  Runs
 * attn_decode_packed (same arguments, split plan, kernel build and output)
 * with kernels that also store timestamps of the device's constant 100 MHz
 * clock per work-group:
 *   stamps  device uint64 [n_seq][n_kv_heads][64][8], 16-byte aligned
 *           (64: the most splits a call makes).  Entries of
 *           work-group (i, h, s): 0 entry, 1 Q codes ready, 2 wave 0's first
 *           tile ready, 3 the first and 4 the last wave's ring done, 5 partial
 *           published (split counter returned; stores issued when the merge
 *           is a second launch), 6 merge or direct output done, 7 flags
 *           (bit 0: this work-group merged the splits, bit 1: a single split
 *           wrote its rows directly); entries a work-group never reached are
 *           0.  A work-group writes its 8 entries once, at its end (it keeps
 *           them on chip meanwhile).  Work-groups past a sequence's end
 *           write nothing.
 * Errors as attn_decode_packed; KVQ_ERR_INVALID for a NULL or misaligned
 * stamps buffer.
 */
int kvq_debug_attn_timeline(const kvq_cache* cache, const float* q, float* out, int n_seq,
                            int n_qtok, int n_q_heads, const int32_t* seg_table, int max_segs,
                            const int32_t* seq_len, int max_seq_len, float sm_scale, int causal,
                            void* workspace, size_t workspace_bytes, uint64_t* stamps,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
