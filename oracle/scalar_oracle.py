"""Scalar pure-Python twin of the TBQ4 oracle, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It restates the same
steps as ``tbq4_oracle`` one value at a time with Python floats (IEEE fp64),
so that the vectorised oracle can be checked against an independent
transcription: identical bytes for the quantiser, agreement to rounding for
attention.  The fp16 rounding of the scale is done here with exact rational
arithmetic (``fractions.Fraction``) rather than with a table
of midpoints, so the two quantisers share no method either.

Source page: "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "Od czego zacząłem" (66-byte block of 128 values: 2-byte scale, 64 bytes
of 4-bit indices; attention in the rotated Hadamard domain).
"""

import math
from fractions import Fraction

_MAGS = [0.125, 0.375, 0.625, 0.9375, 1.25, 1.625, 2.0, 2.75]
_R = float.fromhex("0x1.6a09e667f3bccp-4")
_M64 = (1 << 64) - 1


def signs(seed):
    st = seed & _M64
    words = []
    for _ in range(2):
        st = (st + 0x9E3779B97F4A7C15) & _M64
        z = st
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        words.append(z ^ (z >> 31))
    return [-1.0 if (words[i >> 6] >> (i & 63)) & 1 else 1.0 for i in range(128)]


def _half_from_bits(h):
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    if e == 0:
        return Fraction(m, 1 << 24)
    return Fraction(1024 + m, 1 << 10) * Fraction(2) ** (e - 15)


def _half_round_sqrt_exact(ms):
    """Nearest binary16 to sqrt(ms) for an fp64 ms >= 0, exact, ties to even,
    saturating at 65504: walk the fp16 patterns with exact rationals."""
    ms = Fraction(ms)
    lo, hi = 0, 0x7BFF
    # largest h whose value^2 <= ms (h = 0 when ms is tiny)
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if _half_from_bits(mid) ** 2 <= ms:
            lo = mid
        else:
            hi = mid - 1
    h = lo
    if h == 0x7BFF:
        return h
    a, b = _half_from_bits(h), _half_from_bits(h + 1)
    m2 = ((a + b) / 2) ** 2
    if ms < m2:
        return h
    if ms > m2:
        return h + 1
    return h if h % 2 == 0 else h + 1


def quantize_block(x, seed=0):
    """One block of 128 floats -> 66 bytes (list of ints)."""
    s = signs(seed)
    v = [float(x[i]) * s[i] for i in range(128)]
    h = 1
    while h < 128:
        for i in range(128):
            if i & h == 0:
                a, b = v[i], v[i + h]
                v[i], v[i + h] = a + b, a - b
        h *= 2
    u = [vi * _R for vi in v]
    p = [ui * ui for ui in u]
    h = 64
    while h >= 1:
        for i in range(h):
            p[i] = p[i] + p[i + h]
        h //= 2
    ms = p[0] * 2.0 ** -7
    dbits = _half_round_sqrt_exact(ms)
    d = float(_half_from_bits(dbits))
    # sign-magnitude code: sign bit 3 for negative values, magnitude rank =
    # number of magnitude midpoints (scaled by d) strictly below |u|
    tau = [(_MAGS[k] + _MAGS[k + 1]) / 2.0 for k in range(7)]
    idx = []
    for ui in u:
        m = sum(1 for t in tau if d * t < abs(ui))
        idx.append(m + (8 if ui < 0 else 0))
    out = [dbits & 0xFF, dbits >> 8]
    for j in range(64):
        out.append(idx[2 * j] | (idx[2 * j + 1] << 4))
    return out


_MAGS3 = [0.25, 0.75, 1.375, 2.25]


def quantize_block3(x, seed=0):
    """One block of 128 floats -> 50 TBQ3 bytes (list of ints): the same
    rotation and scale as TBQ4, 3-bit sign-magnitude codes (bit 2 = sign),
    code i at bits 3i .. 3i+2 of the little-endian integer in bytes 2..49,
    built here with Python big-integer arithmetic."""
    s = signs(seed)
    v = [float(x[i]) * s[i] for i in range(128)]
    h = 1
    while h < 128:
        for i in range(128):
            if i & h == 0:
                a, b = v[i], v[i + h]
                v[i], v[i + h] = a + b, a - b
        h *= 2
    u = [vi * _R for vi in v]
    p = [ui * ui for ui in u]
    h = 64
    while h >= 1:
        for i in range(h):
            p[i] = p[i] + p[i + h]
        h //= 2
    dbits = _half_round_sqrt_exact(p[0] * 2.0 ** -7)
    d = float(_half_from_bits(dbits))
    tau = [(_MAGS3[k] + _MAGS3[k + 1]) / 2.0 for k in range(3)]
    big = 0
    for i, ui in enumerate(u):
        code = sum(1 for t in tau if d * t < abs(ui)) + (4 if ui < 0 else 0)
        big |= code << (3 * i)
    return [dbits & 0xFF, dbits >> 8] + list(big.to_bytes(48, "little"))


def dequantize_block(block, seed=0):
    """66 bytes -> 128 floats in the original domain."""
    s = signs(seed)
    block = [int(b) for b in block]
    dbits = block[0] | (block[1] << 8)
    d = float(_half_from_bits(dbits))
    y = []
    for j in range(64):
        byte = block[2 + j]
        for code in (byte & 15, byte >> 4):
            y.append(d * (-_MAGS[code - 8] if code >= 8 else _MAGS[code]))
    h = 1
    while h < 128:
        for i in range(128):
            if i & h == 0:
                a, b = y[i], y[i + h]
                y[i], y[i + h] = a + b, a - b
        h *= 2
    return [s[i] * y[i] * _R for i in range(128)]


def attend(q, keys, values, scale):
    """softmax(scale * q.K^T) V for one query vector, pure Python."""
    s = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in keys]
    m = max(s)
    e = [math.exp(si - m) for si in s]
    z = sum(e)
    return [sum(e[j] * values[j][i] for j in range(len(keys))) / z for i in range(len(q))]
