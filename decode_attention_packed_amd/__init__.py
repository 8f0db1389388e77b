"""Packed-KV decode attention for AMD MI355X (gfx950).

The compute path is libkvq.so (include/kvq.h): hand-written HIP kernels for
quantize-and-append, split-K decode attention and the split combine.  This
package is the thin Python binding over that C ABI; PyTorch provides device
memory and streams only.
"""
from ._lib import (EXPORTS, KVQ_NOALLOC_SCRATCH_BYTES, attn_decode_packed_noalloc, KVQ_BLOCK, KVQ_ERR_HIP, KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED,
                   KVQ_ERR_WORKSPACE, KVQ_MAX_QTOK, KVQ_OK, KVQ_SEG_ALIGN, KVQ_V_Q4_0, KVQ_V_Q8_0,
                   KvqCacheStruct, KvqError, PackedKVCache, attn_decode_packed,
                   attn_decode_packed_append, KVQ_MAX_APPEND, F16KCache, attn_decode_f16k,
                   attn_decode_f16k_workspace_size, kv_append_f16k, kvq_f16k_cache_bytes,
                   attn_decode_packed_batch, attn_decode_packed_batch_workspace_size, KVQ_MAX_BATCH,
                   attn_decode_packed_workspace_size, kv_append_quant, kvq_abi_version,
                   kvq_cache_bytes, kvq_debug_attn_isum, kvq_debug_attn_timeline, kvq_debug_qk_isum, kvq_debug_quant_q, kvq_debug_stream_read, lib,
                   status_string)

__all__ = ["EXPORTS", "KVQ_NOALLOC_SCRATCH_BYTES", "attn_decode_packed_noalloc", "KVQ_BLOCK", "KVQ_ERR_HIP", "KVQ_ERR_INVALID", "KVQ_ERR_UNSUPPORTED",
           "KVQ_ERR_WORKSPACE", "KVQ_MAX_QTOK", "KVQ_OK", "KVQ_SEG_ALIGN", "KVQ_V_Q4_0",
           "KVQ_V_Q8_0", "KvqCacheStruct", "KvqError", "PackedKVCache", "attn_decode_packed",
           "attn_decode_packed_append", "KVQ_MAX_APPEND", "F16KCache", "attn_decode_f16k",
           "attn_decode_f16k_workspace_size", "kv_append_f16k", "kvq_f16k_cache_bytes",
           "attn_decode_packed_batch", "attn_decode_packed_batch_workspace_size", "KVQ_MAX_BATCH",
           "attn_decode_packed_workspace_size", "kv_append_quant", "kvq_abi_version",
           "kvq_cache_bytes", "kvq_debug_attn_isum", "kvq_debug_attn_timeline", "kvq_debug_qk_isum", "kvq_debug_quant_q", "kvq_debug_stream_read", "lib",
           "status_string"]
