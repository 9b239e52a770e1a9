"""Pins of the oracle's q8_0 rows against things other than itself.

The pages name q8_0 as a KV cache type (the tgstat.ru channel @tech_di page's
server configuration sets both cache tensors to it) without defining it; the
oracle reads it as 32-value blocks of a binary16 scale d = amax/127 and int8
codes round(x/d), halves away from zero, decided in fp32.  Checked here:
hand-derived blocks, the scale against an enumeration of binary16 values, the
codes against exact rational arithmetic, and the error bound.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import tbq4_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "known_rows_q8_0.json")) as f:
        return json.load(f)["rows"]


def test_layout():
    assert o.Q8_ROW_BYTES == 4 * (2 + 32) == 136
    assert o.Q8_ROW_BYTES * 8 / o.HEAD_DIM == 8.5
    r = o.q8_0_rows(np.zeros((3, 5, 128), np.float32))
    assert r.shape == (3, 5, 136) and not r.any()


@pytest.mark.parametrize("row", _gold(), ids=lambda r: r["name"])
def test_known_blocks(row):
    x = np.zeros(128, np.float32)
    k = row["block"]
    x[32 * k:32 * k + len(row["values"])] = row["values"]
    got = o.q8_0_rows(x)
    assert got[34 * k:34 * (k + 1)].tobytes().hex() == row["hex"]
    rest = np.delete(got, np.arange(34 * k, 34 * (k + 1)))
    assert not rest.any()


def _fp32_nearest(f):
    """The IEEE binary32 value nearest the rational f, ties to even, found by
    checking the neighbours of a first guess."""
    g = np.float32(float(f))
    cands = [np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - f),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return best


def _half_table():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    return bits, bits.view(np.float16).astype(np.float64)


def test_codes_and_scale_against_exact_arithmetic():
    rng = np.random.default_rng(71)
    x = (rng.standard_normal((300, 128)) * 10.0 ** rng.uniform(-4, 4, size=(300, 1))).astype(np.float32)
    rows = o.q8_0_rows(x)
    q, d = o.unpack_q8_0(rows)
    hbits, hvals = _half_table()
    for i in range(0, 300, 7):
        for k in range(4):
            blk = x[i, 32 * k:32 * (k + 1)]
            amax = max(abs(Fraction(float(v))) for v in blk)
            d32 = _fp32_nearest(amax / 127)
            # the stored scale is the binary16 nearest d32 (ties to even)
            dist = np.abs(hvals - float(d32))
            j = np.flatnonzero(dist == dist.min())
            j = j[hbits[j] % 2 == 0][0] if len(j) > 1 else j[0]
            assert d[i, k] == hvals[j]
            for e, v in enumerate(blk):
                r = _fp32_nearest(Fraction(float(v)) / Fraction(float(d32)))
                a = abs(Fraction(float(r)))
                want = int(a + Fraction(1, 2)) * (1 if r >= 0 else -1)   # floor(|r| + 1/2)
                assert q[i, k, e] == want, (i, k, e)


def test_ties_go_away_from_zero_and_extremes():
    x = np.zeros(128, np.float32)
    x[:6] = [127, 0.5, -0.5, 126.5, -126.5, 1e-3]
    q, d = o.unpack_q8_0(o.q8_0_rows(x))
    assert d[0] == 1.0
    assert list(q[0, :6]) == [127, 1, -1, 127, -127, 0]
    # the largest magnitude always takes code +-127
    rng = np.random.default_rng(72)
    y = rng.standard_normal((200, 128)).astype(np.float32)
    q, _ = o.unpack_q8_0(o.q8_0_rows(y))
    yb = y.reshape(200, 4, 32)
    arg = np.argmax(np.abs(yb), axis=-1)
    top = np.take_along_axis(q, arg[..., None], axis=-1)[..., 0]
    assert np.array_equal(np.abs(top), np.full((200, 4), 127))
    assert np.array_equal(np.sign(top), np.sign(np.take_along_axis(yb, arg[..., None], -1)[..., 0]))


def test_error_bound():
    rng = np.random.default_rng(73)
    x = (rng.standard_t(3, size=(500, 128)) * rng.uniform(0.01, 100, size=(500, 1))).astype(np.float32)
    xh = o.dequantize_q8_0(o.q8_0_rows(x))
    xb = x.reshape(500, 4, 32).astype(np.float64)
    d32 = (np.max(np.abs(x.reshape(500, 4, 32)), axis=-1) / np.float32(127)).astype(np.float64)
    _, d = o.unpack_q8_0(o.q8_0_rows(x))
    bound = 0.5 * d32 * (1 + 2.0 ** -20) + 127.5 * np.abs(d - d32)
    err = np.abs(xh.reshape(500, 4, 32) - xb)
    assert np.all(err <= bound[..., None] + 1e-30)
    rel = np.linalg.norm(xh - x) / np.linalg.norm(x)
    assert rel < 0.01
