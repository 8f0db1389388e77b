"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every step of the path runs in the HIP library; this module checks tensor
dtypes and shapes, passes raw pointers and the current torch stream, and
turns a negative status into KvqError.  PyTorch supplies device memory and
streams and nothing else.  The library must have been built
(decode_attention_packed_amd.build_lib.build()); a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_WORKSPACE = -3
KVQ_ERR_HIP = -4
KVQ_V_Q4_0 = 0
KVQ_V_Q8_0 = 1
KVQ_BLOCK = 32
KVQ_SEG_ALIGN = 64
KVQ_MAX_QTOK = 16
KVQ_MAX_APPEND = 16
KVQ_MAX_BATCH = 4
KVQ_NOALLOC_SCRATCH_BYTES = 8 << 20

EXPORTS = ("kvq_abi_version", "kvq_status_string", "kvq_cache_bytes", "kv_append_quant",
           "attn_decode_packed_append",
           "attn_decode_packed_workspace_size", "attn_decode_packed", "kvq_debug_quant_q",
           "kvq_debug_qk_isum", "kvq_debug_stream_read", "kvq_f16k_cache_bytes", "kv_append_f16k",
           "attn_decode_f16k_workspace_size", "attn_decode_f16k", "attn_decode_packed_batch",
           "attn_decode_packed_batch_workspace_size", "kvq_debug_attn_isum",
           "attn_decode_packed_noalloc", "kvq_debug_attn_timeline")


class KvqCacheStruct(ctypes.Structure):
    _fields_ = [("n_kv_heads", c_int32), ("head_dim", c_int32), ("seg_tokens", c_int32),
                ("n_segs", c_int32), ("v_format", c_int32), ("reserved", c_int32),
                ("k_qs", c_void_p), ("k_d", c_void_p), ("v_qs", c_void_p), ("v_d", c_void_p)]


class KvqAttnCallStruct(ctypes.Structure):
    _fields_ = [("cache", POINTER(KvqCacheStruct)), ("q", c_void_p), ("out", c_void_p),
                ("n_seq", c_int32), ("n_qtok", c_int32), ("n_q_heads", c_int32),
                ("seg_table", c_void_p), ("max_segs", c_int32), ("seq_len", c_void_p),
                ("max_seq_len", c_int32), ("sm_scale", c_float), ("causal", c_int32)]


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvq; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libkvq.so not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = POINTER(KvqCacheStruct)
        L.kvq_abi_version.restype = c_int
        L.kvq_abi_version.argtypes = []
        L.kvq_status_string.restype = c_char_p
        L.kvq_status_string.argtypes = [c_int]
        L.kvq_cache_bytes.restype = c_int
        L.kvq_cache_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, POINTER(c_size_t)]
        L.kv_append_quant.restype = c_int
        L.kv_append_quant.argtypes = [P, c_void_p, c_void_p, c_int, c_int, c_void_p, c_int,
                                      c_void_p, c_void_p]
        L.attn_decode_packed_workspace_size.restype = c_int
        L.attn_decode_packed_workspace_size.argtypes = [P, c_int, c_int, c_int, c_int,
                                                        POINTER(c_size_t)]
        L.attn_decode_packed.restype = c_int
        L.attn_decode_packed.argtypes = [P, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_int,
                                         c_void_p, c_int, c_float, c_int, c_void_p, c_size_t,
                                         c_void_p]
        L.attn_decode_packed_append.restype = c_int
        L.attn_decode_packed_append.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                                c_int, c_int, c_int, c_void_p, c_int, c_void_p,
                                                c_int, c_float, c_int, c_void_p, c_size_t,
                                                c_void_p]
        L.kvq_f16k_cache_bytes.restype = c_int
        L.kvq_f16k_cache_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, POINTER(c_size_t)]
        L.kv_append_f16k.restype = c_int
        L.kv_append_f16k.argtypes = L.kv_append_quant.argtypes
        L.attn_decode_f16k_workspace_size.restype = c_int
        L.attn_decode_f16k_workspace_size.argtypes = L.attn_decode_packed_workspace_size.argtypes
        L.attn_decode_f16k.restype = c_int
        L.attn_decode_f16k.argtypes = L.attn_decode_packed.argtypes
        L.attn_decode_packed_batch_workspace_size.restype = c_int
        L.attn_decode_packed_batch_workspace_size.argtypes = [POINTER(KvqAttnCallStruct), c_int,
                                                              POINTER(c_size_t)]
        L.attn_decode_packed_batch.restype = c_int
        L.attn_decode_packed_batch.argtypes = [POINTER(KvqAttnCallStruct), c_int, c_void_p, c_size_t,
                                               c_void_p]
        L.kvq_debug_stream_read.restype = c_int
        L.kvq_debug_stream_read.argtypes = [c_void_p, ctypes.c_size_t, c_void_p, c_void_p]
        L.kvq_debug_quant_q.restype = c_int
        L.kvq_debug_quant_q.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]
        L.kvq_debug_qk_isum.restype = c_int
        L.kvq_debug_qk_isum.argtypes = [P, c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_void_p,
                                        c_int, c_void_p, c_void_p]
        L.attn_decode_packed_noalloc.restype = c_int
        L.attn_decode_packed_noalloc.argtypes = L.attn_decode_packed.argtypes[:-3] + [c_void_p]
        L.kvq_debug_attn_timeline.restype = c_int
        L.kvq_debug_attn_timeline.argtypes = L.attn_decode_packed.argtypes[:-1] + [c_void_p, c_void_p]
        L.kvq_debug_attn_isum.restype = c_int
        L.kvq_debug_attn_isum.argtypes = L.attn_decode_packed.argtypes[:-1] + [c_void_p, c_void_p]
        if L.kvq_abi_version() != 1:
            raise ImportError("libkvq ABI version mismatch")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, where)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _need(t, dtype, name, ndim=None, device=True):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def kvq_abi_version() -> int:
    return lib().kvq_abi_version()


def kvq_cache_bytes(n_kv_heads: int, head_dim: int, seg_tokens: int, n_segs: int,
                    v_format: int) -> tuple:
    out = (c_size_t * 4)()
    _check(lib().kvq_cache_bytes(n_kv_heads, head_dim, seg_tokens, n_segs, v_format, out),
           "kvq_cache_bytes")
    return tuple(int(x) for x in out)


class PackedKVCache:
    """Caller-owned cache planes (torch device tensors) plus the C struct that
    points at them.  Layout: [n_segs][n_kv_heads][seg_tokens][...] per plane."""

    def __init__(self, n_kv_heads: int, head_dim: int, seg_tokens: int, n_segs: int,
                 v_format: int, device="cuda"):
        import torch
        kq, kd, vq, vd = kvq_cache_bytes(n_kv_heads, head_dim, seg_tokens, n_segs, v_format)
        nb = head_dim // KVQ_BLOCK
        shape = (n_segs, n_kv_heads, seg_tokens)
        self.k_qs = torch.empty(shape + (head_dim // 4,), dtype=torch.int32, device=device)
        self.k_d = torch.empty(shape + (nb,), dtype=torch.int16, device=device)
        vrow = head_dim // 2 if v_format == KVQ_V_Q4_0 else head_dim
        self.v_qs = torch.empty(shape + (vrow,), dtype=torch.uint8, device=device)
        self.v_d = torch.empty(shape + (nb,), dtype=torch.int16, device=device)
        assert (self.k_qs.numel() * 4, self.k_d.numel() * 2, self.v_qs.numel(),
                self.v_d.numel() * 2) == (kq, kd, vq, vd)
        self.n_kv_heads, self.head_dim, self.seg_tokens = n_kv_heads, head_dim, seg_tokens
        self.n_segs, self.v_format = n_segs, v_format
        self.struct = KvqCacheStruct(n_kv_heads, head_dim, seg_tokens, n_segs, v_format, 0,
                                     self.k_qs.data_ptr(), self.k_d.data_ptr(),
                                     self.v_qs.data_ptr(), self.v_d.data_ptr())

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k_qs, self.k_d, self.v_qs, self.v_d))


class F16KCache:
    """The fp16-K A/B cache: K as binary16 rows [n_segs][n_kv_heads][seg_tokens]
    [head_dim] (no K scales), V as in PackedKVCache.  head_dim 128 only."""

    def __init__(self, n_kv_heads: int, head_dim: int, seg_tokens: int, n_segs: int,
                 v_format: int, device="cuda"):
        import torch
        k, kd, vq, vd = kvq_f16k_cache_bytes(n_kv_heads, head_dim, seg_tokens, n_segs, v_format)
        nb = head_dim // KVQ_BLOCK
        shape = (n_segs, n_kv_heads, seg_tokens)
        self.k = torch.empty(shape + (head_dim,), dtype=torch.int16, device=device)
        vrow = head_dim // 2 if v_format == KVQ_V_Q4_0 else head_dim
        self.v_qs = torch.empty(shape + (vrow,), dtype=torch.uint8, device=device)
        self.v_d = torch.empty(shape + (nb,), dtype=torch.int16, device=device)
        assert (self.k.numel() * 2, kd, self.v_qs.numel(), self.v_d.numel() * 2) == (k, 0, vq, vd)
        self.n_kv_heads, self.head_dim, self.seg_tokens = n_kv_heads, head_dim, seg_tokens
        self.n_segs, self.v_format = n_segs, v_format
        self.struct = KvqCacheStruct(n_kv_heads, head_dim, seg_tokens, n_segs, v_format, 0,
                                     self.k.data_ptr(), None, self.v_qs.data_ptr(),
                                     self.v_d.data_ptr())

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k, self.v_qs, self.v_d))


def kvq_f16k_cache_bytes(n_kv_heads: int, head_dim: int, seg_tokens: int, n_segs: int,
                         v_format: int) -> tuple:
    out = (c_size_t * 4)()
    _check(lib().kvq_f16k_cache_bytes(n_kv_heads, head_dim, seg_tokens, n_segs, v_format, out),
           "kvq_f16k_cache_bytes")
    return tuple(int(x) for x in out)


def kv_append_f16k(cache: F16KCache, k_new, v_new, start_pos, seg_table=None,
                   max_segs: int | None = None, stream=None) -> None:
    """kv_append_quant for the fp16-K A/B cache."""
    _append(lib().kv_append_f16k, "kv_append_f16k", cache, k_new, v_new, start_pos, seg_table,
            max_segs, stream)


def attn_decode_f16k_workspace_size(cache: F16KCache, n_seq: int, n_qtok: int, n_q_heads: int,
                                    max_seq_len: int) -> int:
    out = c_size_t(0)
    _check(lib().attn_decode_f16k_workspace_size(ctypes.byref(cache.struct), n_seq, n_qtok,
                                                 n_q_heads, max_seq_len, ctypes.byref(out)),
           "attn_decode_f16k_workspace_size")
    return int(out.value)


def attn_decode_f16k(cache: F16KCache, q, out, seq_len, max_seq_len: int, sm_scale: float,
                     causal: bool, workspace, seg_table=None, max_segs: int | None = None,
                     stream=None) -> None:
    """attn_decode_packed for the fp16-K A/B cache (Q rounded to fp16)."""
    _attend(lib().attn_decode_f16k, "attn_decode_f16k", cache, q, out, seq_len, max_seq_len,
            sm_scale, causal, workspace, seg_table, max_segs, stream)


def kv_append_quant(cache: PackedKVCache, k_new, v_new, start_pos, seg_table=None,
                    max_segs: int | None = None, stream=None) -> None:
    """k_new, v_new: float32 [n_seq][n_new][n_kv_heads][head_dim] on the GPU;
    start_pos: int32 [n_seq]; seg_table: int32 [n_seq][max_segs] or None."""
    _append(lib().kv_append_quant, "kv_append_quant", cache, k_new, v_new, start_pos, seg_table,
            max_segs, stream)


def _append(fn, where, cache, k_new, v_new, start_pos, seg_table, max_segs, stream) -> None:
    import torch
    _need(k_new, torch.float32, "k_new", 4)
    _need(v_new, torch.float32, "v_new", 4)
    _need(start_pos, torch.int32, "start_pos", 1)
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    n_seq, n_new, hkv, d = k_new.shape
    if hkv != cache.n_kv_heads or d != cache.head_dim or start_pos.shape[0] != n_seq:
        raise ValueError("shape does not match the cache")
    if seg_table is not None:
        _need(seg_table, torch.int32, "seg_table", 2)
        max_segs = seg_table.shape[1]
    elif max_segs is None:
        max_segs = cache.n_segs // n_seq
    _check(fn(ctypes.byref(cache.struct), _ptr(k_new), _ptr(v_new), n_seq, n_new,
              _ptr(seg_table), int(max_segs), _ptr(start_pos), _stream(stream)), where)


def attn_decode_packed_workspace_size(cache: PackedKVCache, n_seq: int, n_qtok: int,
                                      n_q_heads: int, max_seq_len: int) -> int:
    out = c_size_t(0)
    _check(lib().attn_decode_packed_workspace_size(ctypes.byref(cache.struct), n_seq, n_qtok,
                                                   n_q_heads, max_seq_len, ctypes.byref(out)),
           "attn_decode_packed_workspace_size")
    return int(out.value)


def attn_decode_packed(cache: PackedKVCache, q, out, seq_len, max_seq_len: int, sm_scale: float,
                       causal: bool, workspace, seg_table=None, max_segs: int | None = None,
                       stream=None) -> None:
    """q, out: float32 [n_seq][n_qtok][n_q_heads][head_dim]; seq_len: int32 [n_seq];
    workspace: a GPU tensor of at least attn_decode_packed_workspace_size bytes."""
    _attend(lib().attn_decode_packed, "attn_decode_packed", cache, q, out, seq_len, max_seq_len,
            sm_scale, causal, workspace, seg_table, max_segs, stream)


def _attend(fn, where, cache, q, out, seq_len, max_seq_len, sm_scale, causal, workspace, seg_table,
            max_segs, stream) -> None:
    import torch
    _need(q, torch.float32, "q", 4)
    _need(out, torch.float32, "out", 4)
    _need(seq_len, torch.int32, "seq_len", 1)
    if q.shape != out.shape:
        raise ValueError("q and out differ in shape")
    n_seq, n_qtok, n_q_heads, d = q.shape
    if d != cache.head_dim or seq_len.shape[0] != n_seq:
        raise ValueError("shape does not match the cache")
    if seg_table is not None:
        _need(seg_table, torch.int32, "seg_table", 2)
        max_segs = seg_table.shape[1]
    elif max_segs is None:
        max_segs = cache.n_segs // n_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(ctypes.byref(cache.struct), _ptr(q), _ptr(out), n_seq, n_qtok, n_q_heads,
              _ptr(seg_table), int(max_segs), _ptr(seq_len), int(max_seq_len), float(sm_scale),
              int(bool(causal)), _ptr(workspace), ws_bytes, _stream(stream)), where)


def attn_decode_packed_append(cache: PackedKVCache, q, k_new, v_new, out, seq_len,
                              max_seq_len: int, sm_scale: float, causal: bool, workspace,
                              seg_table=None, max_segs: int | None = None, stream=None) -> None:
    """Append k_new / v_new (float32 [n_seq][n_new][n_kv_heads][head_dim]) at
    tokens seq_len - n_new .. seq_len - 1 and attend, in one launch; other
    arguments as attn_decode_packed."""
    import torch
    _need(q, torch.float32, "q", 4)
    _need(out, torch.float32, "out", 4)
    _need(k_new, torch.float32, "k_new", 4)
    _need(v_new, torch.float32, "v_new", 4)
    _need(seq_len, torch.int32, "seq_len", 1)
    if q.shape != out.shape:
        raise ValueError("q and out differ in shape")
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    n_seq, n_qtok, n_q_heads, d = q.shape
    if (d != cache.head_dim or seq_len.shape[0] != n_seq or k_new.shape[0] != n_seq
            or k_new.shape[2] != cache.n_kv_heads or k_new.shape[3] != d):
        raise ValueError("shape does not match the cache")
    n_new = k_new.shape[1]
    if seg_table is not None:
        _need(seg_table, torch.int32, "seg_table", 2)
        max_segs = seg_table.shape[1]
    elif max_segs is None:
        max_segs = cache.n_segs // n_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_decode_packed_append(ctypes.byref(cache.struct), _ptr(q), _ptr(k_new),
                                           _ptr(v_new), _ptr(out), n_seq, n_qtok, n_q_heads, n_new,
                                           _ptr(seg_table), int(max_segs), _ptr(seq_len),
                                           int(max_seq_len), float(sm_scale), int(bool(causal)),
                                           _ptr(workspace), ws_bytes, _stream(stream)),
           "attn_decode_packed_append")


def _batch_calls(calls):
    """calls: dicts with cache, q, out, seq_len, max_seq_len, sm_scale, causal
    and optionally seg_table / max_segs, as attn_decode_packed takes them."""
    import torch
    arr = (KvqAttnCallStruct * len(calls))()
    for i, c in enumerate(calls):
        cache, q, out, seq_len = c["cache"], c["q"], c["out"], c["seq_len"]
        _need(q, torch.float32, "q", 4)
        _need(out, torch.float32, "out", 4)
        _need(seq_len, torch.int32, "seq_len", 1)
        if q.shape != out.shape:
            raise ValueError("q and out differ in shape")
        n_seq, n_qtok, n_q_heads, d = q.shape
        if d != cache.head_dim or seq_len.shape[0] != n_seq:
            raise ValueError("shape does not match the cache")
        seg_table = c.get("seg_table")
        if seg_table is not None:
            _need(seg_table, torch.int32, "seg_table", 2)
            max_segs = seg_table.shape[1]
        else:
            max_segs = c.get("max_segs") or cache.n_segs // n_seq
        arr[i] = KvqAttnCallStruct(ctypes.pointer(cache.struct), _ptr(q), _ptr(out), n_seq, n_qtok,
                                   n_q_heads, _ptr(seg_table), int(max_segs), _ptr(seq_len),
                                   int(c["max_seq_len"]), float(c["sm_scale"]), int(bool(c["causal"])))
    return arr


def attn_decode_packed_batch_workspace_size(calls) -> int:
    arr = _batch_calls(calls)
    out = c_size_t(0)
    _check(lib().attn_decode_packed_batch_workspace_size(arr, len(calls), ctypes.byref(out)),
           "attn_decode_packed_batch_workspace_size")
    return int(out.value)


def attn_decode_packed_batch(calls, workspace, stream=None) -> None:
    """Several attn_decode_packed calls (see _batch_calls) in one launch."""
    arr = _batch_calls(calls)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_decode_packed_batch(arr, len(calls), _ptr(workspace), ws_bytes, _stream(stream)),
           "attn_decode_packed_batch")


def kvq_debug_stream_read(buf, sink, stream=None) -> None:
    """Stream-read every byte of the device tensor `buf` (contiguous, size a
    multiple of 16); `sink` is a device int32/uint32 tensor of >= 1 element."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda:
        raise ValueError("buf and sink must be contiguous device tensors")
    _check(lib().kvq_debug_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)),
           "kvq_debug_stream_read")


def kvq_debug_quant_q(q, codes, scales, stream=None) -> None:
    """q float32 [rows][D] -> codes int8 [rows][D], scales float32 [rows][D/32]."""
    import torch
    _need(q, torch.float32, "q", 2)
    _need(codes, torch.int8, "codes", 2)
    _need(scales, torch.float32, "scales", 2)
    _check(lib().kvq_debug_quant_q(_ptr(q), q.shape[0], q.shape[1], _ptr(codes), _ptr(scales),
                                   _stream(stream)), "kvq_debug_quant_q")


def kvq_debug_qk_isum(cache: PackedKVCache, q, seq_len, max_seq_len: int, isum, seg_table=None,
                      max_segs: int | None = None, stream=None) -> None:
    """isum int32 [n_seq][n_qtok][n_q_heads][max_seq_len][D/32]."""
    import torch
    _need(q, torch.float32, "q", 4)
    _need(isum, torch.int32, "isum", 5)
    _need(seq_len, torch.int32, "seq_len", 1)
    n_seq, n_qtok, n_q_heads, _ = q.shape
    if seg_table is not None:
        _need(seg_table, torch.int32, "seg_table", 2)
        max_segs = seg_table.shape[1]
    elif max_segs is None:
        max_segs = cache.n_segs // n_seq
    _check(lib().kvq_debug_qk_isum(ctypes.byref(cache.struct), _ptr(q), n_seq, n_qtok, n_q_heads,
                                   _ptr(seg_table), int(max_segs), _ptr(seq_len), int(max_seq_len),
                                   _ptr(isum), _stream(stream)), "kvq_debug_qk_isum")


def kvq_debug_attn_isum(cache: PackedKVCache, q, out, seq_len, max_seq_len: int, sm_scale: float,
                        causal: bool, workspace, isum, seg_table=None, max_segs: int | None = None,
                        stream=None) -> None:
    """attn_decode_packed that also stores the kernels' per-block int32 Q.K
    sums: isum int32 [n_seq][n_qtok][n_q_heads][max_seq_len][D/32]."""
    import torch
    _need(isum, torch.int32, "isum", 5)
    fn = lib().kvq_debug_attn_isum

    def call(*args):
        return fn(*args[:-1], _ptr(isum), args[-1])
    _attend(call, "kvq_debug_attn_isum", cache, q, out, seq_len, max_seq_len, sm_scale, causal,
            workspace, seg_table, max_segs, stream)


def attn_decode_packed_noalloc(cache: PackedKVCache, q, out, seq_len, max_seq_len: int,
                               sm_scale: float, causal: bool, seg_table=None,
                               max_segs: int | None = None, stream=None) -> None:
    """attn_decode_packed without a workspace argument: the library's static
    device scratch array (KVQ_NOALLOC_SCRATCH_BYTES per GPU) holds the split
    partials; nothing is allocated."""
    fn = lib().attn_decode_packed_noalloc

    def call(*args):
        # drop the workspace pointer and size that _attend passes
        return fn(*args[:-3], args[-1])
    _attend(call, "attn_decode_packed_noalloc", cache, q, out, seq_len, max_seq_len, sm_scale,
            causal, None, seg_table, max_segs, stream)


def kvq_debug_attn_timeline(cache: PackedKVCache, q, out, seq_len, max_seq_len: int,
                            sm_scale: float, causal: bool, workspace, stamps, seg_table=None,
                            max_segs: int | None = None, stream=None) -> None:
    """attn_decode_packed that also stores per-work-group timestamps: stamps
    int64 (read as uint64) [n_seq][n_kv_heads][64][8], contiguous."""
    import torch
    _need(stamps, torch.int64, "stamps")
    fn = lib().kvq_debug_attn_timeline

    def call(*args):
        return fn(*args[:-1], _ptr(stamps), args[-1])
    _attend(call, "kvq_debug_attn_timeline", cache, q, out, seq_len, max_seq_len, sm_scale, causal,
            workspace, seg_table, max_segs, stream)
