"""Pins of the oracle's TBQ3 quantiser against things other than itself.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "6. Ten sam cache na Apple silicon": a TBQ3 KV cache beside TBQ4, and
a fix to its 3-bit packing -- so the packing is tested exhaustively here.
Layout as read in the oracle: 2-byte binary16 scale + 48 bytes of 3-bit codes,
code i at bits 3i .. 3i+2 of the little-endian integer in bytes 2..49.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import scalar_oracle as so
from oracle import tbq4_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _gauss_mse(levels):
    c = np.asarray(levels, np.float64)
    t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    a, b = t[:-1], t[1:]
    m0 = norm.cdf(b) - norm.cdf(a)
    m1 = norm.pdf(a) - norm.pdf(b)
    m2 = m0 + np.where(np.isinf(a), 0.0, a) * norm.pdf(a) - np.where(np.isinf(b), 0.0, b) * norm.pdf(b)
    return float(np.sum(m2 - 2 * c * m1 + c * c * m0))


def test_layout():
    assert o.BLOCK_BYTES3 == 2 + 48
    assert o.BLOCK_BYTES3 * 8 / o.HEAD_DIM == 3.125
    packed, codes, _ = o.quantize_blocks3(np.zeros((2, 128), np.float32))
    assert packed.shape == (2, 50) and codes.shape == (2, 128)


def test_lloyd_max_eight_levels_matches_max_1960():
    g = _gold("max1960_n8.json")
    c = np.linspace(-2, 2, 8)
    for _ in range(2000):
        t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
        c = np.array([(norm.pdf(a) - norm.pdf(b)) / (norm.cdf(b) - norm.cdf(a))
                      for a, b in zip(t[:-1], t[1:])])
    np.testing.assert_allclose(c[4:], g["positive_output_levels"], atol=g["table_precision"])
    np.testing.assert_allclose(((c[:-1] + c[1:]) / 2)[3:], g["positive_thresholds"],
                               atol=g["table_precision"])
    assert abs(_gauss_mse(c) - g["mse"]) < 2e-5


def test_codebook_is_best_four_significant_bit_codebook():
    g = _gold("max1960_n8.json")
    pos = o.MAGNITUDES3
    assert np.array_equal(o.CODEBOOK3, np.concatenate([-pos[::-1], pos]))
    assert np.array_equal(o.MAG_THRESHOLDS3, (pos[:-1] + pos[1:]) / 2)
    for v in pos:                       # <= 4 significant bits: exact in fp16, bf16, e4m3
        m, e = math.frexp(v)
        assert (m * 16) == int(m * 16)

    def grid_near(v):
        return sorted({mant * 2.0 ** (e - 3) for e in range(-6, 4) for mant in range(8, 16)
                       if abs(mant * 2.0 ** (e - 3) - v) <= 0.15 * v + 0.02})
    best = None
    for combo in itertools.product(*[grid_near(v) for v in g["positive_output_levels"]]):
        if np.all(np.diff(combo) > 0):
            m = _gauss_mse(np.concatenate([-np.array(combo)[::-1], combo]))
            if best is None or m < best[0]:
                best = (m, combo)
    assert tuple(pos) == tuple(best[1])
    assert g["mse"] < _gauss_mse(o.CODEBOOK3) < 1.02 * g["mse"]


def test_packing_every_code_at_every_position():
    """A single code c at position i, zeros elsewhere, is the integer c << 3i
    of the 48 little-endian bytes (Python big integers, not the numpy path)."""
    for i in range(128):
        for c in range(8):
            codes = np.zeros(128, np.uint8)
            codes[i] = c
            b = o.pack3(codes)
            assert int.from_bytes(b.tobytes(), "little") == c << (3 * i), (i, c)
            assert np.array_equal(o.unpack3(b), codes)


def test_packing_random_blocks_and_roundtrip():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 8, size=(200, 128)).astype(np.uint8)
    packed = o.pack3(codes)
    for row, b in zip(codes, packed):
        assert int.from_bytes(b.tobytes(), "little") == sum(int(c) << (3 * i) for i, c in enumerate(row))
    assert np.array_equal(o.unpack3(packed), codes)
    # every byte boundary inside the stream is crossed by some code
    crossing = [i for i in range(128) if (3 * i) // 8 != (3 * i + 2) // 8]
    assert len(crossing) == 32


@pytest.mark.parametrize("blk", _gold("known_blocks_tbq3.json")["blocks"], ids=lambda b: b["name"])
def test_known_answer_blocks(blk):
    x = np.zeros(128)
    if blk["input"]["kind"] == "unit":
        x[blk["input"]["index"]] = blk["input"]["scale"]
    assert o.quantize_blocks3(x, blk["seed"])[0].tobytes().hex() == blk["hex"]
    assert bytes(so.quantize_block3(x, blk["seed"])).hex() == blk["hex"]


def test_code_is_nearest_level_ties_toward_zero():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((300, 128)) * rng.uniform(0.01, 100, size=(300, 1))
    _, codes, d_bits = o.quantize_blocks3(x.astype(np.float32))
    u = o.rotate(x.astype(np.float32).astype(np.float64), o.sign_vector(0))
    d = o.half_bits_to_float(d_bits)
    lv = np.array([v for m in o.MAGNITUDES3 for v in (m, -m)])     # smaller magnitude, + first
    nearest = lv[np.argmin(np.abs(u[..., None] - d[:, None, None] * lv), axis=-1)]
    assert np.array_equal(o.CODE_VALUES3[codes] * d[:, None], nearest * d[:, None])
    assert np.array_equal(codes >= 4, u < 0)
    # exact midpoints take the smaller magnitude, u = 0 takes +0.25
    dd = 0.5
    for k, t in enumerate(o.MAG_THRESHOLDS3):
        assert int((dd * o.MAG_THRESHOLDS3 < dd * t).sum()) == k
    assert np.all(o.quantize_blocks3(np.zeros(128))[1] == 0)


def test_scale_is_the_tbq4_scale_and_scalar_twin_agrees():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((40, 128)) * rng.uniform(0.001, 1000, size=(40, 1))).astype(np.float32)
    p3, _, d3 = o.quantize_blocks3(x, 7)
    _, _, d4 = o.quantize_blocks(x, 7)
    assert np.array_equal(d3, d4)
    for row, blk in zip(x, p3):
        assert bytes(so.quantize_block3(row, 7)) == blk.tobytes()


def test_roundtrip_error_matches_codebook_mse():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((4000, 128))
    p, _, _ = o.quantize_blocks3(x, 0)
    xh = o.dequantize_blocks3(p, 0)
    rel = np.mean((xh - x) ** 2) / np.mean(x ** 2)
    # per-block RMS scaling on Gaussian blocks sits near the N(0,1) MSE
    assert abs(rel - _gauss_mse(o.CODEBOOK3)) < 0.003
    # dequantised rotated values are exactly d * level
    idx, d = o.unpack_blocks3(p[:5])
    assert np.array_equal(o.dequantize_rotated3(p[:5]), d[:, None] * o.CODE_VALUES3[idx])
