"""Plain, slow, fp64 CPU oracle for TBQ4 attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares
no code, tables or constants with the HIP library; every constant below is
written out here independently.

What it computes, and where that comes from
-------------------------------------------
Source page: "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq"
(trefon.com notes).

* Section "Od czego zacząłem": a TBQ4 block holds 128 values in 66 bytes -- a
  2-byte scale followed by 64 bytes of 4-bit indices (4.125 bits per value) --
  and attention runs in the rotated (Hadamard) domain, with dequantisation in
  the inner loop and no F16 buffer.
* Section "Konfiguracja": both the K and the V cache use the ``tbq4_0`` type
  (``-ctk tbq4_0 -ctv tbq4_0``), flash attention is on.
* Section "Liczby": 4.125 bpv and about 4.1 GiB at 262144 tokens.

The page does not fix the rotation's sign vector, the codebook, the scale
statistic, the rounding rules or the nibble order.  The readings taken here
(each one is listed with its reason in the design notes of the repository):

* rotation   u = R x,  R = H D / sqrt(128): D = diag(s) with s a +-1 vector
               drawn from SplitMix64(seed), H the natural-order Sylvester
               Hadamard matrix (H_ij = (-1)^popcount(i&j)); signs first.
* scale      d = the binary16 value nearest the exact square root of the mean
               square of u, ties to even, saturating at 65504.
* codebook   16 sign-symmetric levels: of all sign-symmetric 16-level
               codebooks whose levels have at most 4 significant bits, the one
               with least mean-square error on N(0,1) under nearest-level
               decisions (the 16-level Lloyd-Max quantiser held to a grid on
               which every level is exact in fp16, bf16 and fp8 e4m3).
* code       each value becomes a 4-bit sign-magnitude code, laid out like
               the 4-bit e2m1 float: bit 3 = sign (set for u_i < 0), bits 0-2
               = m_i = #{k in 0..6 : d * tau_k < |u_i|}, tau_k the midpoints of
               adjacent magnitudes.  This picks the nearest level; a value
               exactly between two magnitudes takes the smaller one, and
               u_i = 0 takes +0.125 d (so an all-zero block packs to zeros).
* pack       bytes 0-1 = d (binary16, little endian); byte 2+j holds the code
               of element 2j in its low nibble and of element 2j+1 in its high
               nibble.
* attention  plain softmax attention on the dequantised cache; query head h
               reads KV head floor(h / G), G = H_q / H_kv; a prefill query at
               absolute position n_past+i attends keys 0..n_past+i inclusive.

Every floating-point step of the quantiser is an IEEE-754 fp64 operation in a
stated order, so the packed bytes are a deterministic function of the input.
"""

import numpy as np

HEAD_DIM = 128
BLOCK_BYTES = 66
_MASK64 = (1 << 64) - 1

# --------------------------------------------------------------------------
# Codebook: the least-MSE sign-symmetric 16-level quantiser of N(0,1) whose
# levels have at most four significant bits (it sits next to the 16-level
# Lloyd-Max levels 0.1284 ... 2.733).  CODEBOOK lists the levels in ascending
# order; a 4-bit code (s, m) stands for (-1)^s * MAGNITUDES[m].
# --------------------------------------------------------------------------
MAGNITUDES = np.array([0.125, 0.375, 0.625, 0.9375, 1.25, 1.625, 2.0, 2.75], dtype=np.float64)
CODEBOOK = np.concatenate([-MAGNITUDES[::-1], MAGNITUDES])
THRESHOLDS = (CODEBOOK[:-1] + CODEBOOK[1:]) / 2.0          # 15 values, exact
MAG_THRESHOLDS = (MAGNITUDES[:-1] + MAGNITUDES[1:]) / 2.0  # 7 values, exact
# value of each 4-bit code 0..15
CODE_VALUES = np.concatenate([MAGNITUDES, -MAGNITUDES])

# fl64(1/sqrt(128)) -- the normalisation of the 128-point transform.
INV_SQRT128 = float.fromhex("0x1.6a09e667f3bccp-4")


# --------------------------------------------------------------------------
# Sign vector: SplitMix64 (Steele, Lea and Flood, "Fast splittable
# pseudorandom number generators", OOPSLA 2014).
# --------------------------------------------------------------------------
def splitmix64(seed, n):
    """First ``n`` outputs of SplitMix64 started from ``seed`` (ints < 2**64)."""
    state = seed & _MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_bits(seed):
    """The 16 bytes of the sign vector: bit i (little endian) set <=> s_i = -1."""
    w0, w1 = splitmix64(seed, 2)
    return w0.to_bytes(8, "little") + w1.to_bytes(8, "little")


def sign_vector(seed):
    """s in {+1,-1}^128: s_i = -1 iff bit (i mod 64) of word floor(i/64) is 1."""
    w = splitmix64(seed, 2)
    s = np.ones(HEAD_DIM, dtype=np.float64)
    for i in range(HEAD_DIM):
        if (w[i // 64] >> (i % 64)) & 1:
            s[i] = -1.0
    return s


# --------------------------------------------------------------------------
# Walsh-Hadamard transform (natural order), fp64 butterflies.
# --------------------------------------------------------------------------
def _butterfly(v):
    """In order h = 1, 2, ..., 64: (v_i, v_{i+h}) <- (v_i + v_{i+h}, v_i - v_{i+h})
    for every i with (i & h) == 0.  Returns H v (unnormalised)."""
    v = np.array(v, dtype=np.float64, copy=True)
    lead = v.shape[:-1]
    h = 1
    while h < HEAD_DIM:
        w = v.reshape(lead + (HEAD_DIM // (2 * h), 2, h))
        a = w[..., 0, :]
        b = w[..., 1, :]
        v = np.stack((a + b, a - b), axis=-2).reshape(lead + (HEAD_DIM,))
        h *= 2
    return v


def rotate(x, signs):
    """u = R x = H (s * x) * fl64(1/sqrt(128)), along the last axis, in fp64."""
    v = np.asarray(x, dtype=np.float64) * signs
    return _butterfly(v) * INV_SQRT128


def unrotate(y, signs):
    """x = R^T y = s * (H y) * fl64(1/sqrt(128)); R^T R = I because H H = 128 I."""
    return signs * (_butterfly(np.asarray(y, dtype=np.float64)) * INV_SQRT128)


# --------------------------------------------------------------------------
# binary16 helpers
# --------------------------------------------------------------------------
def _half_values():
    bits = np.arange(0x7C00, dtype=np.uint16)          # +0 ... 65504
    return bits.view(np.float16).astype(np.float64)


_HALF_VALUES = _half_values()
# mid2[h-1] = ((value(h-1) + value(h)) / 2)^2 for h = 1..0x7BFF.  A midpoint
# has at most 12 significant bits, so its square is exact in fp64.
_MID2 = ((_HALF_VALUES[:-1] + _HALF_VALUES[1:]) / 2.0) ** 2


def half_nearest_sqrt(ms):
    """binary16 bit pattern of the value nearest sqrt(ms) (exact real root),
    ties to even, saturating at 65504 (0x7BFF).  ``ms`` is an fp64 array >= 0.

    The pattern h is the number of midpoints below sqrt(ms) -- counting a
    midpoint equal to sqrt(ms) only when the pattern above it is even -- so
    the comparison is between exact squares and never takes a square root."""
    ms = np.asarray(ms, dtype=np.float64)
    n_lt = np.searchsorted(_MID2, ms, side="left")
    n_le = np.searchsorted(_MID2, ms, side="right")
    tie = n_le > n_lt                       # sqrt(ms) is exactly midpoint n_lt+1
    take_tie = tie & (((n_lt + 1) % 2) == 0)
    return (n_lt + take_tie).astype(np.uint16)


def half_bits_to_float(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Quantiser
# --------------------------------------------------------------------------
def _rotate_and_scale(x, seed):
    """The steps TBQ4 and TBQ3 share: u = R x in fp64 and the binary16 scale
    d nearest sqrt(mean u^2).  Returns (u, d_bits, d)."""
    signs = sign_vector(seed)
    x = np.asarray(x)
    if x.shape[-1] != HEAD_DIM:
        raise ValueError("last axis must be 128")
    u = rotate(x.astype(np.float64), signs)

    # mean square: p_i = u_i*u_i, then the tree p_i += p_{i+h} for
    # h = 64, 32, ..., 1 and i < h; S = p_0; ms = S * 2^-7 (exact).
    p = u * u
    h = HEAD_DIM // 2
    while h >= 1:
        p = p.copy()
        p[..., :h] = p[..., :h] + p[..., h:2 * h]
        h //= 2
    ms = p[..., 0] * (2.0 ** -7)

    d_bits = half_nearest_sqrt(ms)
    return u, d_bits, half_bits_to_float(d_bits)


def quantize_blocks(x, seed=0):
    """Quantise blocks of 128 values to TBQ4.

    x: array (..., 128) in fp32 / fp16 / fp64 (converted to fp64 exactly).
    Returns (packed uint8 (..., 66), codes uint8 (..., 128), d_bits uint16 (...)).
    """
    x = np.asarray(x)
    u, d_bits, d = _rotate_and_scale(x, seed)

    # code = sign bit | number of scaled magnitude thresholds below |u|
    # (d * tau_k is exact in fp64)
    thr = d[..., None] * MAG_THRESHOLDS                   # (..., 7)
    mag = (thr[..., None, :] < np.abs(u)[..., :, None]).sum(axis=-1)
    idx = (mag + 8 * (u < 0)).astype(np.uint8)

    packed = np.empty(x.shape[:-1] + (BLOCK_BYTES,), dtype=np.uint8)
    packed[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    packed[..., 1] = (d_bits >> 8).astype(np.uint8)
    packed[..., 2:] = idx[..., 0::2] | (idx[..., 1::2] << 4)
    return packed, idx, d_bits


def unpack_blocks(packed):
    """Inverse of the byte layout: returns (codes uint8 (..., 128), d fp64 (...))."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.shape[-1] != BLOCK_BYTES:
        raise ValueError("last axis must be 66 bytes")
    d_bits = packed[..., 0].astype(np.uint16) | (packed[..., 1].astype(np.uint16) << 8)
    q = packed[..., 2:]
    idx = np.empty(packed.shape[:-1] + (HEAD_DIM,), dtype=np.uint8)
    idx[..., 0::2] = q & 0x0F
    idx[..., 1::2] = q >> 4
    return idx, half_bits_to_float(d_bits)


def dequantize_rotated(packed):
    """y = d * value(code): the block's values in the rotated domain (fp64, exact)."""
    idx, d = unpack_blocks(packed)
    return d[..., None] * CODE_VALUES[idx]


def dequantize_blocks(packed, seed=0):
    """x_hat = R^T (d * c[idx]) in fp64: the block in the original domain."""
    return unrotate(dequantize_rotated(packed), sign_vector(seed))


# --------------------------------------------------------------------------
# TBQ3: the same method with 3-bit codes.  The page "Kontekst 262K na jednej
# RTX 4090: co dodałem do llama.cpp-turboq", section "6. Ten sam cache na
# Apple silicon", names a TBQ3 KV cache beside TBQ4 (with a fix to its 3-bit
# packing) and rotated-domain dequantisation in attention for both; the TBQ3
# layout is not given.  Reading
# (the plainest one consistent with TBQ4): 128 values -> a 2-byte binary16
# scale (the same RMS rule) + 48 bytes of 3-bit codes = 50 bytes, 3.125 bits
# per value; the same rotation; the least-MSE sign-symmetric 8-level
# quantiser of N(0,1) whose levels have at most four significant bits; a code
# is sign-magnitude (bit 2 set for u < 0, bits 0-1 the magnitude index = the
# number of scaled magnitude midpoints below |u|: nearest level, ties toward
# zero, u = 0 -> +0.25); code i occupies bits 3i .. 3i+2 of the 384-bit
# little-endian integer held in bytes 2..49 (codes cross byte boundaries).
# --------------------------------------------------------------------------
BLOCK_BYTES3 = 50
MAGNITUDES3 = np.array([0.25, 0.75, 1.375, 2.25], dtype=np.float64)
CODEBOOK3 = np.concatenate([-MAGNITUDES3[::-1], MAGNITUDES3])
MAG_THRESHOLDS3 = (MAGNITUDES3[:-1] + MAGNITUDES3[1:]) / 2.0   # 0.5, 1.0625, 1.8125
CODE_VALUES3 = np.concatenate([MAGNITUDES3, -MAGNITUDES3])     # value of code 0..7


def pack3(codes):
    """codes uint8 (..., 128) in 0..7 -> (..., 48) bytes: code i at bits
    3i .. 3i+2 of the little-endian bit string."""
    codes = np.asarray(codes, dtype=np.uint8)
    bits = (codes[..., :, None] >> np.arange(3, dtype=np.uint8)) & 1      # (..., 128, 3)
    bits = bits.reshape(codes.shape[:-1] + (3 * HEAD_DIM,))
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack3(packed48):
    bits = np.unpackbits(np.asarray(packed48, dtype=np.uint8), axis=-1, bitorder="little")
    bits = bits.reshape(bits.shape[:-1] + (HEAD_DIM, 3))
    return (bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)).astype(np.uint8)


def quantize_blocks3(x, seed=0):
    """Quantise blocks of 128 values to TBQ3.  Returns (packed uint8 (..., 50),
    codes uint8 (..., 128), d_bits uint16 (...))."""
    x = np.asarray(x)
    u, d_bits, d = _rotate_and_scale(x, seed)
    thr = d[..., None] * MAG_THRESHOLDS3                  # exact in fp64
    mag = (thr[..., None, :] < np.abs(u)[..., :, None]).sum(axis=-1)
    idx = (mag + 4 * (u < 0)).astype(np.uint8)
    packed = np.empty(x.shape[:-1] + (BLOCK_BYTES3,), dtype=np.uint8)
    packed[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    packed[..., 1] = (d_bits >> 8).astype(np.uint8)
    packed[..., 2:] = pack3(idx)
    return packed, idx, d_bits


def unpack_blocks3(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.shape[-1] != BLOCK_BYTES3:
        raise ValueError("last axis must be 50 bytes")
    d_bits = packed[..., 0].astype(np.uint16) | (packed[..., 1].astype(np.uint16) << 8)
    return unpack3(packed[..., 2:]), half_bits_to_float(d_bits)


def dequantize_rotated3(packed):
    idx, d = unpack_blocks3(packed)
    return d[..., None] * CODE_VALUES3[idx]


def dequantize_blocks3(packed, seed=0):
    return unrotate(dequantize_rotated3(packed), sign_vector(seed))


# --------------------------------------------------------------------------
# fp16 cache rows (mixed K/V cache formats).  Page "Kontekst 262K na jednej
# RTX 4090: co dodałem do llama.cpp-turboq", section "Konfiguracja": the K and
# V cache types are chosen separately; the plain alternative to TBQ4 is an fp16
# cache.  A head vector is stored as 128 IEEE binary16 values, each the
# binary16 nearest to the input (ties to even; beyond the largest finite value
# it overflows to infinity), not rotated.
# --------------------------------------------------------------------------
def f16_rows(x):
    """IEEE binary16 of every element (numpy's float32 -> float16 cast rounds
    to nearest even; the fp32 input is exact in float32)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def dequantize_f16(rows):
    return np.asarray(rows, dtype=np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# q8_0 cache rows (mixed K/V cache formats).  The pages name q8_0 as a KV cache
# type (the tgstat.ru channel @tech_di page: its server configuration sets
# both the K and the V cache to q8_0; the DFlash speed-test page weighs a
# quantised cache against fp16) but never define it.  Read here as the common
# 8-bit block format: each head vector is four blocks of 32 values; a block
# is its binary16 scale d (little endian) followed by 32 int8 codes, 34 bytes,
# 136 bytes per head vector, not rotated.  Decisions are made in IEEE fp32,
# the precision of the kernel:
#   amax = max |x_i| (exact),  d32 = amax / 127 (fp32, nearest even),
#   q_i  = x_i / d32 (fp32, nearest even) rounded to the nearest integer,
#          halves away from zero; q_i = 0 when d32 = 0,
#   d    = the binary16 nearest d32 (ties to even).
# A code's value is d * q_i.  (Inputs are finite.)
# --------------------------------------------------------------------------
Q8_BLOCK = 32
Q8_BLOCK_BYTES = 34
Q8_ROW_BYTES = 136


def q8_0_rows(x):
    """Head vectors (..., 128) -> q8_0 rows uint8 (..., 136)."""
    x32 = np.asarray(x, dtype=np.float32)
    xb = x32.reshape(x32.shape[:-1] + (HEAD_DIM // Q8_BLOCK, Q8_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (xb / d32[..., None]).astype(np.float32)
    av = np.floor(np.abs(v.astype(np.float64)) + 0.5)
    q = np.where(d32[..., None] > 0, np.where(v < 0, -av, av), 0.0).astype(np.int8)
    rows = np.empty(x32.shape[:-1] + (HEAD_DIM // Q8_BLOCK, Q8_BLOCK_BYTES), dtype=np.uint8)
    d_bits = d32.astype(np.float16).view(np.uint16)
    rows[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    rows[..., 1] = (d_bits >> 8).astype(np.uint8)
    rows[..., 2:] = q.view(np.uint8)
    return rows.reshape(x32.shape[:-1] + (Q8_ROW_BYTES,))


def unpack_q8_0(rows):
    """q8_0 rows (..., 136) -> (codes int8 (..., 4, 32), d fp64 (..., 4))."""
    rows = np.asarray(rows, dtype=np.uint8)
    if rows.shape[-1] != Q8_ROW_BYTES:
        raise ValueError("last axis must be 136 bytes")
    b = rows.reshape(rows.shape[:-1] + (HEAD_DIM // Q8_BLOCK, Q8_BLOCK_BYTES))
    d_bits = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
    return b[..., 2:].view(np.int8), half_bits_to_float(d_bits)


def dequantize_q8_0(rows):
    q, d = unpack_q8_0(rows)
    x = d[..., None] * q.astype(np.float64)
    return x.reshape(x.shape[:-2] + (HEAD_DIM,))


# --------------------------------------------------------------------------
# Attention on the dequantised cache (plain softmax attention, fp64)
# --------------------------------------------------------------------------
def _softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attn_decode_ref(q, k_cache, v_cache, n_ctx, softmax_scale, seed=0):
    """One decode query per (sequence, head).

    q:       (B, H_q, 128) float
    k_cache: (B, H_kv, cap, 66) uint8 packed TBQ4 blocks (same for v_cache)
    Returns o: (B, H_q, 128) fp64.  Query head h reads KV head h // (H_q/H_kv);
    keys 0..n_ctx-1 are attended.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            K = dequantize_blocks(k_cache[b, g, :n_ctx], seed)     # (n_ctx, 128)
            V = dequantize_blocks(v_cache[b, g, :n_ctx], seed)
            Q = q[b, g * G:(g + 1) * G]                            # (G, 128)
            p = _softmax_rows(softmax_scale * (Q @ K.T))
            out[b, g * G:(g + 1) * G] = p @ V
    return out


def attn_decode_rotated_ref(q, k_cache, v_cache, n_ctx, softmax_scale, seed=0):
    """The same decode attention taken in the rotated domain:
    q' = R q;  s_j = scale * (q' . y^K_j);  o' = sum_j p_j y^V_j;  o = R^T o'."""
    signs = sign_vector(seed)
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            Yk = dequantize_rotated(k_cache[b, g, :n_ctx])
            Yv = dequantize_rotated(v_cache[b, g, :n_ctx])
            Qr = rotate(q[b, g * G:(g + 1) * G], signs)
            p = _softmax_rows(softmax_scale * (Qr @ Yk.T))
            out[b, g * G:(g + 1) * G] = unrotate(p @ Yv, signs)
    return out


def attn_decode_rows_ref(q_rows, K, V, softmax_scale):
    """Decode attention for a few query rows against dequantised K, V (fp64):
    q_rows (r, 128), K and V (n, 128).  Used when only some heads are checked."""
    p = _softmax_rows(softmax_scale * (np.asarray(q_rows, np.float64) @ K.T))
    return p @ V


def attn_prefill_rows_ref(q_rows, K, V, n_past, rows, softmax_scale, chunk=64):
    """Causal prefill attention for some query rows of one KV-head group,
    against dequantised K, V (fp64).

    q_rows (r, G, 128): the G query heads of chunk queries ``rows`` (r
    indices); K, V (n, 128) with n >= n_past + max(rows) + 1.  Query i sits at
    absolute position n_past + i and attends keys 0 .. n_past + i: its scores
    against later keys are -inf before the softmax (weight exactly 0).  Rows
    are taken ``chunk`` at a time so that K is read once per chunk.  Returns
    (r, G, 128)."""
    q_rows = np.asarray(q_rows, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    r, G, D = q_rows.shape
    out = np.empty((r, G, D), dtype=np.float64)
    for c0 in range(0, r, chunk):
        idx = rows[c0:c0 + chunk]
        n_keys = n_past + idx + 1                          # keys each row sees
        top = int(n_keys.max())
        s = softmax_scale * (q_rows[c0:c0 + chunk].reshape(-1, D) @ K[:top].T)
        s = s.reshape(len(idx), G, top)
        s = np.where(np.arange(top)[None, None, :] < n_keys[:, None, None], s, -np.inf)
        out[c0:c0 + chunk] = _softmax_rows(s) @ V[:top]
    return out


def attn_prefill_ref(q, k_cache, v_cache, n_past, softmax_scale, seed=0,
                     rows=None, kv_heads=None):
    """Causal prefill-chunk attention.

    q: (B, n_q, H_q, 128).  Query i sits at absolute position n_past + i and
    attends keys 0..n_past+i of its KV head (the chunk's own K/V must already
    be in the cache).  ``rows`` optionally restricts the query indices and
    ``kv_heads`` the KV heads that are computed (others are left NaN).
    Returns (B, n_q, H_q, 128) fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, n_q, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    n_tot = n_past + n_q
    out = np.full((B, n_q, Hq, D), np.nan)
    for b in range(B):
        for g in kv_heads:
            K = dequantize_blocks(k_cache[b, g, :n_tot], seed)
            V = dequantize_blocks(v_cache[b, g, :n_tot], seed)
            for i in rows:
                n_keys = n_past + int(i) + 1
                Q = q[b, i, g * G:(g + 1) * G]                     # (G, 128)
                p = _softmax_rows(softmax_scale * (Q @ K[:n_keys].T))
                out[b, i, g * G:(g + 1) * G] = p @ V[:n_keys]
    return out


# --------------------------------------------------------------------------
# Split-K (flash-decoding) partials and their log-sum-exp merge.
# --------------------------------------------------------------------------
def split_partials(s, V, bounds):
    """Partial softmax state per key range: for each [a, b) in ``bounds``
    returns (m, l, acc) with m = max s, l = sum exp(s - m), acc = sum exp(s - m) V."""
    parts = []
    for a, b in bounds:
        m = s[a:b].max()
        e = np.exp(s[a:b] - m)
        parts.append((m, e.sum(), e @ V[a:b]))
    return parts


def merge_partials(parts):
    """o = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p, M = max_p m_p."""
    M = max(m for m, _, _ in parts)
    l = sum(np.exp(m - M) * lp for m, lp, _ in parts)
    acc = sum(np.exp(m - M) * ap for m, _, ap in parts)
    return acc / l
