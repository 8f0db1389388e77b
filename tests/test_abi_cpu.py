"""Host-side checks of the C ABI: the library loads, exports every function
include/kvq.h declares, sizes caches by the closed form, and rejects bad
arguments before touching the GPU (none of these calls reaches HIP)."""
import ctypes
import os
import re

import pytest

import decode_attention_packed_amd as K
from decode_attention_packed_amd._lib import KvqCacheStruct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "attn_decode_packed" in names and "kv_append_quant" in names
    L = K.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(K.EXPORTS) == names


def test_abi_version_and_status_strings():
    assert K.kvq_abi_version() == 1
    assert K.status_string(0) == "ok"
    assert K.status_string(K.KVQ_ERR_WORKSPACE) == "workspace too small"
    assert K.status_string(12345) == "unknown status"


def test_cache_bytes_closed_form():
    kq, kd, vq, vd = K.kvq_cache_bytes(8, 128, 131072, 1, K.KVQ_V_Q4_0)
    rows = 8 * 131072
    assert (kq, kd, vq, vd) == (rows * 128, rows * 8, rows * 64, rows * 8)
    # K bytes per element: 34 per 32 -> 1 - 34/64 = 46.875% below fp16 (the 47% of page 1)
    assert 1 - (kq + kd) / (rows * 128 * 2) == 1 - 34 / 64
    kq, kd, vq, vd = K.kvq_cache_bytes(32, 64, 4096, 35, K.KVQ_V_Q8_0)
    assert vq == 35 * 32 * 4096 * 64 and vd == kd
    with pytest.raises(K.KvqError):
        K.kvq_cache_bytes(8, 100, 64, 1, 0)
    with pytest.raises(K.KvqError):
        K.kvq_cache_bytes(8, 128, 64, 1, 7)


def _fake_cache(**kw):
    args = dict(n_kv_heads=8, head_dim=128, seg_tokens=1024, n_segs=1, v_format=0, reserved=0,
                k_qs=0x1000, k_d=0x2000, v_qs=0x3000, v_d=0x4000)
    args.update(kw)
    return KvqCacheStruct(**args)


def _attn(c, q=0x5000, out=0x6000, n_seq=1, n_qtok=1, hq=32, table=None, max_segs=1,
          seq_len=0x7000, max_len=1024, scale=0.1, ws=0x8000, ws_bytes=1 << 30):
    L = K.lib()
    return L.attn_decode_packed(ctypes.byref(c), q, out, n_seq, n_qtok, hq, table, max_segs, seq_len,
                                max_len, scale, 0, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), K.KVQ_ERR_UNSUPPORTED),
    (dict(head_dim=100), K.KVQ_ERR_INVALID),
    (dict(seg_tokens=100), K.KVQ_ERR_INVALID),
    (dict(v_format=3), K.KVQ_ERR_INVALID),
    (dict(reserved=1), K.KVQ_ERR_INVALID),
    (dict(k_qs=0x1004), K.KVQ_ERR_INVALID),
    (dict(v_d=None), K.KVQ_ERR_INVALID),
    (dict(n_kv_heads=0), K.KVQ_ERR_INVALID),
])
def test_bad_cache_rejected(kw, status):
    assert _attn(_fake_cache(**kw)) == status


def test_bad_attention_args_rejected():
    c = _fake_cache()
    assert _attn(c, hq=12) == K.KVQ_ERR_INVALID              # not a multiple of n_kv_heads
    assert _attn(c, hq=8 * 17) == K.KVQ_ERR_UNSUPPORTED      # 17 rows per kv head
    assert _attn(c, n_qtok=17) == K.KVQ_ERR_INVALID
    assert _attn(c, n_qtok=5) == K.KVQ_ERR_UNSUPPORTED        # 5 tokens x 4 heads > 16
    assert _attn(c, max_len=2048) == K.KVQ_ERR_INVALID       # beyond max_segs * seg_tokens
    assert _attn(c, n_seq=2) == K.KVQ_ERR_INVALID            # no table and too few segments
    assert _attn(c, q=0x5008) == K.KVQ_ERR_INVALID           # misaligned
    assert _attn(c, seq_len=None) == K.KVQ_ERR_INVALID
    assert _attn(c, scale=float("nan")) == K.KVQ_ERR_INVALID
    assert _attn(c, ws_bytes=16) == K.KVQ_ERR_WORKSPACE
    assert _attn(c, ws=None) == K.KVQ_ERR_WORKSPACE
    # empty calls are rejected before any launch, not run as no-ops
    assert _attn(c, n_seq=0) == K.KVQ_ERR_INVALID
    assert _attn(c, n_qtok=0) == K.KVQ_ERR_INVALID
    assert _attn(c, max_len=0) == K.KVQ_ERR_INVALID


def test_workspace_size_is_host_only():
    c = _fake_cache(seg_tokens=131072)
    out = ctypes.c_size_t(0)
    assert K.lib().attn_decode_packed_workspace_size(ctypes.byref(c), 1, 1, 32, 131072,
                                                      ctypes.byref(out)) == 0
    assert out.value > 0 and out.value % 4 == 0
    assert K.lib().attn_decode_packed_workspace_size(ctypes.byref(c), 1, 1, 30, 131072,
                                                      ctypes.byref(out)) == K.KVQ_ERR_INVALID


def _r256(x):
    return (x + 255) // 256 * 256


def _splits_from_workspace(c, n_seq, n_qtok, hq, max_len):
    """The split count the planner chose, read back from the workspace size
    (256-byte counters, then [groups][splits][rows][D] partial rows, then their (m, l))."""
    out = ctypes.c_size_t(0)
    assert K.lib().attn_decode_packed_workspace_size(ctypes.byref(c), n_seq, n_qtok, hq, max_len,
                                                      ctypes.byref(out)) == 0
    groups = n_seq * c.n_kv_heads
    rows = n_qtok * (hq // c.n_kv_heads)
    hits = [s for s in range(1, 65)
            if _r256(groups * 256) + _r256(groups * s * rows * c.head_dim * 4) + _r256(groups * s * rows * 8)
            == out.value]
    assert len(hits) == 1, (out.value, hits)
    return hits[0]


@pytest.mark.parametrize("hkv,d,n_seq,hq,max_len,want", [
    (1, 128, 1, 4, 512, 1),         # short sequence, few groups: one split, no merge
    (1, 128, 1, 4, 1024, 4),        # from 1024 tokens: 256-token splits
    (8, 128, 1, 32, 8192, 32),      # gqa8k: about 256 work-groups
    (8, 128, 1, 32, 131072, 32),    # the 128k step: 4096-token chunks
    (8, 128, 1, 32, 131073, 32),    # one token more: still 32 splits (4128 tokens), not 33
    (8, 128, 1, 32, 100000, 32),    # any length: one work-group per CU
    (4, 128, 1, 16, 131072, 64),    # the verify step's draft cache alone
    (16, 128, 2, 32, 50000, 8),     # 32 groups: 8 splits
    (8, 128, 8, 32, 131072, 8),     # 64 groups: at least 8 splits per sequence
    (8, 128, 8, 32, 131073, 8),     # one token more: still 8 (even chunks), not 9
    (16, 128, 16, 32, 32769, 2),    # 256 groups one token past 32k: two even splits
    (32, 64, 16, 32, 32768, 1),     # ragged: 512 groups, unsplit
    (16, 128, 16, 32, 32768, 2),    # 256 groups: the longest sequence in two
    (4, 128, 75, 8, 4096, 1),       # 300 groups: unsplit
])
def test_split_plan(hkv, d, n_seq, hq, max_len, want):
    """The split planner's rules, pinned through the workspace size (host
    only): about one work-group per CU for few groups with at least 8 splits
    per sequence, no split for sequences of at most 512 tokens, and at most
    two (sequence, kv head) groups' worth of work-groups per CU for wide
    batches."""
    c = _fake_cache(n_kv_heads=hkv, head_dim=d, seg_tokens=(max_len + 63) // 64 * 64)
    assert _splits_from_workspace(c, n_seq, 1, hq, max_len) == want


def test_bad_append_args_rejected():
    c = _fake_cache()
    L = K.lib()
    f = L.kv_append_quant
    assert f(ctypes.byref(c), None, 0x2000, 1, 1, None, 1, 0x3000, None) == K.KVQ_ERR_INVALID
    assert f(ctypes.byref(c), 0x1000, 0x2000, 0, 1, None, 1, 0x3000, None) == K.KVQ_ERR_INVALID
    assert f(ctypes.byref(c), 0x1000, 0x2000, 2, 1, None, 1, 0x3000, None) == K.KVQ_ERR_INVALID
    assert f(ctypes.byref(c), 0x1000, 0x2000, 1, 1, None, 1, 0x3002, None) == K.KVQ_ERR_INVALID
    assert f(ctypes.byref(_fake_cache(head_dim=256)), 0x1000, 0x2000, 1, 1, None, 1, 0x3000,
             None) == K.KVQ_ERR_UNSUPPORTED


def test_bad_fused_append_args_rejected():
    c = _fake_cache()
    L = K.lib()

    def call(k_new=0x9000, v_new=0xA000, n_new=1, **kw):
        a = dict(q=0x5000, out=0x6000, n_seq=1, n_qtok=1, hq=32, table=None, max_segs=1,
                 seq_len=0x7000, max_len=1024, scale=0.1, ws=0x8000, ws_bytes=1 << 30)
        a.update(kw)
        return L.attn_decode_packed_append(ctypes.byref(c), a["q"], k_new, v_new, a["out"],
                                           a["n_seq"], a["n_qtok"], a["hq"], n_new, a["table"],
                                           a["max_segs"], a["seq_len"], a["max_len"], a["scale"], 0,
                                           a["ws"], a["ws_bytes"], None)

    assert call(k_new=None) == K.KVQ_ERR_INVALID
    assert call(v_new=0xA004) == K.KVQ_ERR_INVALID            # misaligned
    assert call(n_new=0) == K.KVQ_ERR_INVALID
    assert call(n_new=K.KVQ_MAX_APPEND + 1) == K.KVQ_ERR_INVALID
    assert call(n_new=4, max_len=2) == K.KVQ_ERR_INVALID      # more new rows than tokens
    assert call(hq=12) == K.KVQ_ERR_INVALID                   # the attention checks still apply
    assert call(ws_bytes=16) == K.KVQ_ERR_WORKSPACE


def test_f16k_reference_args_rejected():
    """The fp16-K A/B entry points: K rows without a scale plane (k_d NULL),
    head_dim 128 only, column-layout shapes only; validation before launch."""
    L = K.lib()
    c = _fake_cache(k_d=None)

    def attn(cache=c, n_qtok=1, hq=32, ws_bytes=1 << 30):
        return L.attn_decode_f16k(ctypes.byref(cache), 0x5000, 0x6000, 1, n_qtok, hq, None, 1, 0x7000,
                                  1024, 0.1, 0, 0x8000, ws_bytes, None)

    assert attn(cache=_fake_cache()) == K.KVQ_ERR_INVALID              # a packed cache (k_d set)
    assert attn(cache=_fake_cache(k_d=None, head_dim=64)) == K.KVQ_ERR_UNSUPPORTED
    assert attn(n_qtok=2) == K.KVQ_ERR_UNSUPPORTED                      # 8 rows x 4 blocks > 16
    assert attn(ws_bytes=16) == K.KVQ_ERR_WORKSPACE
    assert L.kv_append_f16k(ctypes.byref(_fake_cache()), 0x9000, 0xA000, 1, 1, None, 1, 0x7000,
                            None) == K.KVQ_ERR_INVALID
    out = (ctypes.c_size_t * 4)()
    assert L.kvq_f16k_cache_bytes(8, 128, 1024, 2, 0, out) == K.KVQ_OK
    assert tuple(out) == (2 * 8 * 1024 * 256, 0, 2 * 8 * 1024 * 64, 2 * 8 * 1024 * 8)
    n = ctypes.c_size_t(0)
    assert L.attn_decode_f16k_workspace_size(ctypes.byref(c), 1, 1, 32, 1024, ctypes.byref(n)) == K.KVQ_OK
    assert n.value > 0


def test_batch_args_rejected():
    """attn_decode_packed_batch validates every call and the batch before any
    launch: one head_dim, V format and MFMA layout for all calls."""
    L = K.lib()
    c128 = _fake_cache()
    c64 = _fake_cache(head_dim=64)
    cq8 = _fake_cache(v_format=1)

    def call(cache, n_qtok=1, hq=32):
        return K._lib.KvqAttnCallStruct(ctypes.pointer(cache), 0x5000, 0x6000, 1, n_qtok, hq, None, 1,
                                        0x7000, 1024, 0.1, 0)

    def run(calls, ws_bytes=1 << 30):
        arr = (K._lib.KvqAttnCallStruct * max(1, len(calls)))(*calls)
        return L.attn_decode_packed_batch(arr, len(calls), 0x8000, ws_bytes, None)

    def size(calls):
        arr = (K._lib.KvqAttnCallStruct * max(1, len(calls)))(*calls)
        n = ctypes.c_size_t(0)
        return L.attn_decode_packed_batch_workspace_size(arr, len(calls), ctypes.byref(n)), n.value

    assert run([]) == K.KVQ_ERR_INVALID
    assert run([call(c128)] * (K.KVQ_MAX_BATCH + 1)) == K.KVQ_ERR_INVALID
    assert run([call(c128), call(c64)]) == K.KVQ_ERR_UNSUPPORTED        # head_dim differs
    assert run([call(c128), call(cq8)]) == K.KVQ_ERR_UNSUPPORTED        # V format differs
    assert run([call(c128), call(c128, n_qtok=4)]) == K.KVQ_ERR_UNSUPPORTED   # layouts differ
    assert run([call(c128), call(c128, hq=12)]) == K.KVQ_ERR_INVALID    # a bad call
    st, one = size([call(c128)])
    assert st == K.KVQ_OK and one > 0
    st, two = size([call(c128), call(c128, hq=16)])
    assert st == K.KVQ_OK and two > one
    assert run([call(c128), call(c128, hq=16)], ws_bytes=two - 16) == K.KVQ_ERR_WORKSPACE


def _ws_bytes(c, n_seq, n_qtok, hq, splits):
    """Workspace bytes of one call under a given split count (256-byte
    counters, then the partial rows, then their (m, l), each part rounded)."""
    groups = n_seq * c.n_kv_heads
    rows = n_qtok * (hq // c.n_kv_heads)
    return (_r256(groups * 256) + _r256(groups * splits * rows * c.head_dim * 4)
            + _r256(groups * splits * rows * 8))


@pytest.mark.parametrize("max_len,splits", [
    (131072, 21),   # the verify step: 21 splits of 6272 tokens (252 work-groups), not 20 + a short one
    (40000, 21),    # 1920-token chunks: long enough for the 12-wave kernels (1536 and up)
    (3000, 12),     # short caches: 256-token chunks
])
def test_batch_joint_plan(max_len, splits):
    """The joint split plan of a batched launch with fewer than 256 groups:
    one chunk for both calls of the verify step (main 32/8 heads and draft
    16/4, 4 causal query tokens), the shortest whole number of tiles that
    keeps the grid within 256 work-groups, pinned through the batch's
    workspace size (host only)."""
    main = _fake_cache(n_kv_heads=8, seg_tokens=(max_len + 63) // 64 * 64)
    draft = _fake_cache(n_kv_heads=4, seg_tokens=(max_len + 63) // 64 * 64)

    def call(cache, hq):
        return K._lib.KvqAttnCallStruct(ctypes.pointer(cache), 0x5000, 0x6000, 1, 4, hq, None, 1,
                                        0x7000, max_len, 0.1, 1)
    arr = (K._lib.KvqAttnCallStruct * 2)(call(main, 32), call(draft, 16))
    n = ctypes.c_size_t(0)
    assert K.lib().attn_decode_packed_batch_workspace_size(arr, 2, ctypes.byref(n)) == K.KVQ_OK
    assert n.value == _ws_bytes(main, 1, 4, 32, splits) + _ws_bytes(draft, 1, 4, 16, splits)


def _noalloc(c, q=0x5000, out=0x6000, n_seq=1, n_qtok=1, hq=32, table=None, max_segs=1,
             seq_len=0x7000, max_len=1024, scale=0.1):
    return K.lib().attn_decode_packed_noalloc(ctypes.byref(c), q, out, n_seq, n_qtok, hq, table,
                                              max_segs, seq_len, max_len, scale, 0, None)


def test_noalloc_rejects_before_any_launch():
    """The allocation-free variant checks its arguments as attn_decode_packed
    does, and refuses a call whose workspace would not fit the static scratch
    array, all before it asks the runtime for anything."""
    c = _fake_cache()
    assert K.KVQ_NOALLOC_SCRATCH_BYTES == 8 << 20
    assert _noalloc(c, hq=12) == K.KVQ_ERR_INVALID
    assert _noalloc(c, n_qtok=5) == K.KVQ_ERR_UNSUPPORTED
    assert _noalloc(c, q=0x5008) == K.KVQ_ERR_INVALID
    assert _noalloc(c, scale=float("inf")) == K.KVQ_ERR_INVALID
    assert _noalloc(c, n_seq=0) == K.KVQ_ERR_INVALID
    # 128 sequences x 8 kv heads x 16 query rows x head_dim 128, unsplit:
    # 8 MiB of partials alone, over the limit
    size = ctypes.c_size_t(0)
    assert K.lib().attn_decode_packed_workspace_size(ctypes.byref(c), 128, 4, 32, 1024,
                                                     ctypes.byref(size)) == 0
    assert size.value > K.KVQ_NOALLOC_SCRATCH_BYTES
    assert _noalloc(c, n_seq=128, n_qtok=4, table=0x9000) == K.KVQ_ERR_WORKSPACE
