"""Oracle for packed-KV decode attention: a plain, slow CPU reference.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call
this module; only the test suite, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library.

What it computes (sources are the web pages the method comes from):

* "Flash Attention for llama.cpp on RDNA3 ... Part 1" (page 1), summary and
  first body paragraph: K is kept as an 8-bit payload, four values per
  32-bit word, plus an fp16 scale, and is re-packed as tokens are written;
  QK^T then runs as packed int8 dot products.  The body and the two KLD
  tables use q4_0 and q8_0 for V.
* The 47% K saving in that page's title fixes the block: 32 int8 values and
  one fp16 scale (34 bytes against 64 bytes of fp16).
* "BitLLM" summary (page 3), section "how to use": nibbles are placed so
  that each byte holds two aligned 4-bit values (lane-interleaved packing);
  section "how it differs": KV lives in append-only segments.

The pages leave the exact rounding rules open; the readings taken here are:
the K and q8_0 scale is the fp32 quotient amax/127 rounded to fp16 (nearest,
ties to even); codes are the fp32 quotient x/d rounded to the nearest
integer (ties to even) and clamped to [-127, 127]; the q4_0 scale is m/(-8)
with m the first element of largest magnitude, rounded to fp16, and the
nibble is the rounded quotient plus 8 clamped to [0, 15]; byte j of a q4_0
block holds element j in its low nibble and element j+16 in its high
nibble; Q is quantized the same way as K but keeps its scale in fp32.

Every fp32 step is done with numpy float32 arithmetic, which is IEEE-754
correctly rounded, so one division here is one correctly rounded fp32
division.  Attention itself is the plain two-pass softmax definition in
float64 on the dequantized values, with no splitting and no online
rescaling.

Pins (tests under tests/ marked "not gpu"): nearest-half brute force over
all 65536 binary16 values; exact rational arg-min over all codes for the
quantizers; the round-trip bound, per element against its own block's scale
on rows whose blocks differ in magnitude by 10-10^6 (head_dim 64 and 128);
hand-derived worked blocks and the 47% closed form under tests/golden/; a
50-digit mpmath evaluation of the whole decode step from the raw cache bytes
at head_dim 32, 64 and 128 (one, two and four blocks per row, block scales an
order of magnitude apart, four query heads per kv head, causal and not, both
V formats); softmax invariants for the attention.  A dequantizer that paired
an element with another block's scale fails both the round-trip and the
mpmath pins.  No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
BLOCK = 32          # elements per quantization block along head_dim
V_Q4_0 = 0
V_Q8_0 = 1


# ---------------------------------------------------------------------------
# binary16 helpers
# ---------------------------------------------------------------------------

def half_bits(x) -> np.ndarray:
    """fp32 -> IEEE-754 binary16 bit pattern, round to nearest, ties to even.

    numpy's float32->float16 cast is used as the rounding step; the test
    suite pins it against a brute-force nearest search over every binary16
    value (subnormals and the overflow threshold included)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=F32).astype(np.float16).view(np.uint16)


def half_value(bits) -> np.ndarray:
    """binary16 bit pattern -> exact fp32 value."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(F32)


def _blocks(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=F32)
    d = x.shape[-1]
    if d % BLOCK:
        raise ValueError("head_dim must be a multiple of 32")
    return x.reshape(x.shape[:-1] + (d // BLOCK, BLOCK))


def _rounded_quotient(xb: np.ndarray, d: np.ndarray) -> np.ndarray:
    """round-to-nearest-even of the fp32 quotient x/d (d broadcast per block);
    blocks with d == 0 give 0."""
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = (xb / d[..., None]).astype(F32)
    r = np.rint(qf)
    return np.where(d[..., None] == 0, F32(0), r)


# ---------------------------------------------------------------------------
# quantizers (page 1 summary/body; 32-blocks from the 47% figure)
# ---------------------------------------------------------------------------

def quantize_k(x):
    """K (and q8_0 V) block quantizer.

    Per 32-block: a = max |x|; d = fp16(fl32(a / 127)); c = clamp(rne(fl32(x / d)),
    -127, 127), all codes 0 when d == 0.
    Returns (codes int8 [..., D], scale bits uint16 [..., D/32])."""
    xb = _blocks(x)
    a = np.max(np.abs(xb), axis=-1)
    d32 = (a / F32(127)).astype(F32)
    d_bits = half_bits(d32)
    d = half_value(d_bits)
    c = np.clip(_rounded_quotient(xb, d), -127, 127)
    return c.astype(np.int8).reshape(np.shape(x)), d_bits


def quantize_v_q4_0(x):
    """q4_0 V block quantizer.

    Per 32-block: m = the first element of largest magnitude; d = fp16(fl32(m / -8));
    n = clamp(rne(fl32(x / d)) + 8, 0, 15), all nibbles 8 when d == 0.
    Returns (nibbles uint8 [..., D] in element order, scale bits uint16)."""
    xb = _blocks(x)
    j = np.argmax(np.abs(xb), axis=-1)
    m = np.take_along_axis(xb, j[..., None], axis=-1)[..., 0]
    d32 = (m / F32(-8)).astype(F32)
    d_bits = half_bits(d32)
    d = half_value(d_bits)
    n = np.clip(_rounded_quotient(xb, d) + 8, 0, 15)
    n = np.where(d[..., None] == 0, F32(8), n)
    return n.astype(np.uint8).reshape(np.shape(x)), d_bits


def quantize_q(x):
    """Q block quantizer used before the integer dot (page 1: the dot
    instruction consumes int8 on both sides).  Same as quantize_k, except the
    scale stays fp32: d = fl32(a / 127).
    Returns (codes int8 [..., D], scales float32 [..., D/32])."""
    xb = _blocks(x)
    a = np.max(np.abs(xb), axis=-1)
    d = (a / F32(127)).astype(F32)
    c = np.clip(_rounded_quotient(xb, d), -127, 127)
    return c.astype(np.int8).reshape(np.shape(x)), d


# ---------------------------------------------------------------------------
# storage encodings
# ---------------------------------------------------------------------------

def pack_k(codes) -> np.ndarray:
    """four int8 codes per 32-bit word; byte k of word w is element 4w+k."""
    c = np.asarray(codes, dtype=np.int8)
    u = c.astype(np.uint8).astype(np.uint32)
    u = u.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4))
    return (u[..., 0] | (u[..., 1] << 8) | (u[..., 2] << 16) | (u[..., 3] << 24)).astype(np.uint32)


def unpack_k(words) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint32)
    parts = [((w >> (8 * k)) & 0xFF).astype(np.uint8) for k in range(4)]
    u = np.stack(parts, axis=-1).reshape(w.shape[:-1] + (w.shape[-1] * 4,))
    return u.view(np.int8)


def pack_q4_0(nibbles) -> np.ndarray:
    """per 32-block: byte j (0..15) = nibble j | nibble (j+16) << 4."""
    n = np.asarray(nibbles, dtype=np.uint8)
    nb = n.reshape(n.shape[:-1] + (n.shape[-1] // BLOCK, BLOCK))
    by = (nb[..., :16] | (nb[..., 16:] << 4)).astype(np.uint8)
    return by.reshape(n.shape[:-1] + (n.shape[-1] // 2,))


def unpack_q4_0(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    pb = p.reshape(p.shape[:-1] + (p.shape[-1] // 16, 16))
    n = np.concatenate([pb & 0x0F, pb >> 4], axis=-1)
    return n.reshape(p.shape[:-1] + (p.shape[-1] * 2,))


def encode_k(x):
    """fp32 K rows -> (packed words uint32 [..., D/4], scale bits uint16 [..., D/32])."""
    c, d = quantize_k(x)
    return pack_k(c), d


def encode_v(x, v_format: int):
    """fp32 V rows -> (payload bytes uint8 [..., D/2 or D], scale bits uint16)."""
    if v_format == V_Q4_0:
        n, d = quantize_v_q4_0(x)
        return pack_q4_0(n), d
    if v_format == V_Q8_0:
        c, d = quantize_k(x)
        return c.view(np.uint8), d
    raise ValueError("unknown V format")


# ---------------------------------------------------------------------------
# dequantization (float64, exact: codes times an fp16/fp32 scale)
# ---------------------------------------------------------------------------

def _expand(d, reps):
    return np.repeat(np.asarray(d, dtype=np.float64), reps, axis=-1)


def dequant_k(words, d_bits) -> np.ndarray:
    c = unpack_k(words).astype(np.float64)
    return c * _expand(half_value(d_bits), BLOCK)


def dequant_v(payload, d_bits, v_format: int) -> np.ndarray:
    if v_format == V_Q4_0:
        v = unpack_q4_0(payload).astype(np.float64) - 8.0
    elif v_format == V_Q8_0:
        v = np.asarray(payload, dtype=np.uint8).view(np.int8).astype(np.float64)
    else:
        raise ValueError("unknown V format")
    return v * _expand(half_value(d_bits), BLOCK)


def dequant_q(codes, d) -> np.ndarray:
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * _expand(d, BLOCK)


# ---------------------------------------------------------------------------
# integer dot sums (page 1: QK^T as packed int8 dot products)
# ---------------------------------------------------------------------------

def block_isum(q_codes, k_codes) -> np.ndarray:
    """per 32-block sum of int8 x int8 products, exact in int64; broadcasts
    over leading axes.  Returns int64 [..., D/32]."""
    qc = np.asarray(q_codes, dtype=np.int8).astype(np.int64)
    kc = np.asarray(k_codes, dtype=np.int8).astype(np.int64)
    prod = qc * kc
    return prod.reshape(prod.shape[:-1] + (prod.shape[-1] // BLOCK, BLOCK)).sum(axis=-1)


# ---------------------------------------------------------------------------
# attention (plain definition, float64)
# ---------------------------------------------------------------------------

def softmax_attention(q_hat, k_hat, v_hat, sm_scale: float, n_visible) -> np.ndarray:
    """out[r] = sum_t softmax_t(sm_scale * q_hat[r] . k_hat[t]) v_hat[t] over
    the first n_visible[r] tokens (two passes: max, then exp/sum/normalize).

    q_hat [R, D], k_hat [L, D], v_hat [L, D] float64; n_visible [R] ints >= 1."""
    q_hat = np.asarray(q_hat, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    s = (q_hat @ k_hat.T) * float(sm_scale)
    L = k_hat.shape[0]
    vis = np.asarray(n_visible).reshape(-1, 1)
    s = np.where(np.arange(L)[None, :] < vis, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / np.sum(e, axis=1, keepdims=True)
    return p @ v_hat


def visible_tokens(seq_len: int, n_qtok: int, causal: bool) -> np.ndarray:
    """Tokens seen by each query token.  With a causal mask, query j of the
    n_qtok newest tokens sits at position seq_len - n_qtok + j and sees
    positions 0..that position; otherwise every query sees seq_len tokens."""
    if causal:
        return np.arange(seq_len - n_qtok + 1, seq_len + 1)
    return np.full(n_qtok, seq_len)


def decode_attention(q, k_words, k_d, v_payload, v_d, v_format: int, seq_len,
                     sm_scale: float, causal: bool, q_heads=None) -> np.ndarray:
    """Full decode-attention step from the packed cache.

    q         float32 [S][Tq][Hq][D]
    k_words   uint32  [S][Hkv][Lmax][D/4]   (per-sequence logical token order)
    k_d       uint16  [S][Hkv][Lmax][D/32]
    v_payload uint8   [S][Hkv][Lmax][D/2 | D]
    v_d       uint16  [S][Hkv][Lmax][D/32]
    seq_len   ints [S]; tokens at or after seq_len[i] are ignored.
    Query head h reads kv head h // (Hq/Hkv) (contiguous GQA groups).
    q_heads: optional list of query heads to compute (others left NaN).
    Returns float64 [S][Tq][Hq][D]."""
    q = np.asarray(q, dtype=F32)
    S, Tq, Hq, D = q.shape
    Hkv = k_words.shape[1]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    heads = range(Hq) if q_heads is None else q_heads
    out = np.full((S, Tq, Hq, D), np.nan)
    qc, qd = quantize_q(q)
    q_hat = dequant_q(qc, qd)
    for i in range(S):
        L = int(seq_len[i])
        vis = visible_tokens(L, Tq, causal)
        for kvh in sorted({h // G for h in heads}):
            k_hat = dequant_k(k_words[i, kvh, :L], k_d[i, kvh, :L])
            v_hat = dequant_v(v_payload[i, kvh, :L], v_d[i, kvh, :L], v_format)
            for h in heads:
                if h // G != kvh:
                    continue
                out[i, :, h, :] = softmax_attention(q_hat[i, :, h, :], k_hat, v_hat, sm_scale, vis)
    return out


def decode_attention_f16k(q, k_bits, v_payload, v_d, v_format: int, seq_len, sm_scale: float,
                          causal: bool, q_heads=None) -> np.ndarray:
    """Attention of the fp16-K reference that page 1 compares its packed K
    against (an A/B reference, not the method): K kept as binary16 rows, Q
    rounded to binary16, the dot of the two exact fp16 values, V dequantized
    as in decode_attention.

    k_bits    uint16 [S][Hkv][Lmax][D]  binary16 bit patterns
    other arguments and the result as decode_attention."""
    q = np.asarray(q, dtype=F32)
    S, Tq, Hq, D = q.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    heads = range(Hq) if q_heads is None else q_heads
    out = np.full((S, Tq, Hq, D), np.nan)
    q_hat = half_value(half_bits(q)).astype(np.float64)
    for i in range(S):
        L = int(seq_len[i])
        vis = visible_tokens(L, Tq, causal)
        for kvh in sorted({h // G for h in heads}):
            k_hat = half_value(k_bits[i, kvh, :L]).astype(np.float64)
            v_hat = dequant_v(v_payload[i, kvh, :L], v_d[i, kvh, :L], v_format)
            for h in heads:
                if h // G != kvh:
                    continue
                out[i, :, h, :] = softmax_attention(q_hat[i, :, h, :], k_hat, v_hat, sm_scale, vis)
    return out


def kv_bytes_per_token_head(head_dim: int, v_format: int):
    """(K bytes, V bytes) one token of one kv head occupies: payload plus one
    fp16 scale per 32-block."""
    nb = head_dim // BLOCK
    k = head_dim + 2 * nb
    v = (head_dim // 2 if v_format == V_Q4_0 else head_dim) + 2 * nb
    return k, v
