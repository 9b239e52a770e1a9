"""Pins of the oracle's quantiser against things other than itself.

Block format: page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Od czego zacząłem" (128 values -> 2-byte scale +
64 bytes of 4-bit indices), sections "Konfiguracja" and "Liczby" (4.125 bpv,
about 4.1 GiB at 262144 tokens vs 16 GiB in FP16).
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
from scipy.integrate import quad
from scipy.stats import norm

from oracle import scalar_oracle as so
from oracle import tbq4_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- layout
def test_layout_closed_form():
    g = _gold("layout.json")
    assert g["scale_bytes"] + g["index_bytes"] == g["block_bytes"] == o.BLOCK_BYTES
    assert g["values_per_block"] == o.HEAD_DIM
    assert g["index_bytes"] * 8 == 4 * g["values_per_block"]
    assert o.BLOCK_BYTES * 8 / o.HEAD_DIM == g["bits_per_value"]
    packed, idx, d = o.quantize_blocks(np.zeros((3, 128), np.float32))
    assert packed.shape == (3, 66) and packed.dtype == np.uint8
    # footprints printed on the page, with 128 (layer, kv head) pairs
    gib = 1 << 30
    tbq4 = g["context_tokens"] * 128 * 2 * o.BLOCK_BYTES / gib
    fp16 = g["context_tokens"] * 128 * 2 * 128 * 2 / gib
    assert tbq4 == 4.125 and round(tbq4, 1) == g["tbq4_gib_printed"]
    assert fp16 == g["fp16_gib_printed"]


# ---------------------------------------------------------------- signs
def test_splitmix64_published_outputs():
    g = _gold("splitmix64_seed0.json")
    got = o.splitmix64(g["seed"], len(g["outputs_hex"]))
    assert [f"{w:016x}" for w in got] == g["outputs_hex"]


def test_sign_vector_bits():
    s = o.sign_vector(0)
    w0 = int(_gold("splitmix64_seed0.json")["outputs_hex"][0], 16)
    w1 = int(_gold("splitmix64_seed0.json")["outputs_hex"][1], 16)
    for i in range(128):
        w = w0 if i < 64 else w1
        assert (s[i] < 0) == bool((w >> (i % 64)) & 1)
    assert s[0] == -1.0 and int((s < 0).sum()) == bin(w0).count("1") + bin(w1).count("1")
    assert o.sign_bits(0) == w0.to_bytes(8, "little") + w1.to_bytes(8, "little")
    assert so.signs(0) == list(s)


# ---------------------------------------------------------------- WHT
def test_butterfly_is_sylvester_hadamard():
    """The butterfly equals scipy's natural-order Sylvester Hadamard, exactly
    on integer inputs."""
    H = scipy.linalg.hadamard(128).astype(np.float64)
    i = np.arange(128)
    pop = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(H, (-1.0) ** pop)
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, size=(20, 128)).astype(np.float64)
    assert np.array_equal(o._butterfly(x), x @ H.T)
    assert np.array_equal(H @ H, 128 * np.eye(128))


def test_rotation_orthogonal():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128))
    s = o.sign_vector(0)
    u = o.rotate(x, s)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    np.testing.assert_allclose(o.unrotate(u, s), x, atol=1e-14)
    R = scipy.linalg.hadamard(128) @ np.diag(s) / math.sqrt(128)
    np.testing.assert_allclose(u, x @ R.T, atol=1e-13)
    np.testing.assert_allclose(R @ R.T, np.eye(128), atol=1e-14)


# ---------------------------------------------------------------- scale rounding
def _half_exact(ms):
    return so._half_round_sqrt_exact(ms)


def test_half_sqrt_rounding_exact_rational():
    rng = np.random.default_rng(3)
    ms = np.concatenate([
        10.0 ** rng.uniform(-16, 9.7, size=400),
        np.array([0.0, 2.0 ** -50, 2.0 ** -50 * 1.0000001, 2.0 ** -48, 1.0, 1 / 128,
                  65504.0 ** 2, 65519.9 ** 2, 65520.0 ** 2, 1e12]),
    ])
    got = o.half_nearest_sqrt(ms)
    want = np.array([_half_exact(float(m)) for m in ms], dtype=np.uint16)
    assert np.array_equal(got, want)
    # and against numpy's own fp16 conversion away from rounding boundaries
    ref = np.minimum(np.float16(np.sqrt(ms[:400])).view(np.uint16), 0x7BFF)
    assert (got[:400] == ref).mean() > 0.99


def test_half_sqrt_ties_to_even():
    vals = o._HALF_VALUES
    for h in (1, 2, 3, 100, 101, 0x3C00, 0x3C01, 0x5555, 0x7BFE, 0x7BFF):
        mid = (vals[h - 1] + vals[h]) / 2
        ms = mid * mid                      # exact in fp64
        got = int(o.half_nearest_sqrt(np.array([ms]))[0])
        assert got == (h if h % 2 == 0 else h - 1), h
        assert got == _half_exact(ms)
    # saturation above the largest finite binary16
    assert int(o.half_nearest_sqrt(np.array([1e30]))[0]) == 0x7BFF


# ---------------------------------------------------------------- codebook
def _gauss_mse(levels):
    """Mean-square error of the nearest-level quantiser with these levels on
    N(0,1), from the Gaussian's truncated moments (closed form)."""
    c = np.asarray(levels, np.float64)
    t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    a, b = t[:-1], t[1:]
    m0 = norm.cdf(b) - norm.cdf(a)
    m1 = norm.pdf(a) - norm.pdf(b)
    aa = np.where(np.isinf(a), 0.0, a)
    bb = np.where(np.isinf(b), 0.0, b)
    m2 = m0 + aa * norm.pdf(a) - bb * norm.pdf(b)
    return float(np.sum(m2 - 2 * c * m1 + c * c * m0))


def _sym(pos):
    pos = np.asarray(pos, np.float64)
    return np.concatenate([-pos[::-1], pos])


def test_lloyd_max_recomputed_matches_max_1960():
    """Lloyd conditions on the Gaussian (levels = centroids of cells bounded by
    midpoints) reproduce Max's published table, and the closed-form MSE agrees
    with numerical integration."""
    g = _gold("max1960_n16.json")
    c = np.linspace(-3, 3, 16)
    for _ in range(500):
        t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
        c = np.array([(norm.pdf(a) - norm.pdf(b)) / (norm.cdf(b) - norm.cdf(a))
                      for a, b in zip(t[:-1], t[1:])])
    np.testing.assert_allclose(c[8:], g["positive_output_levels"], atol=g["table_precision"])
    np.testing.assert_allclose(((c[:-1] + c[1:]) / 2)[7:], g["positive_thresholds"],
                               atol=g["table_precision"])
    assert abs(_gauss_mse(c) - g["mse"]) < 1e-5
    t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    num = sum(quad(lambda x, ck=ck: (x - ck) ** 2 * norm.pdf(x), a, b)[0]
              for ck, a, b in zip(c, t[:-1], t[1:]))
    assert abs(num - _gauss_mse(c)) < 1e-9


def test_codebook_is_best_four_significant_bit_codebook():
    g = _gold("max1960_n16.json")
    pos = o.CODEBOOK[8:]
    assert np.array_equal(o.CODEBOOK[:8], -pos[::-1])
    assert np.array_equal(o.THRESHOLDS, (o.CODEBOOK[:-1] + o.CODEBOOK[1:]) / 2)
    # every level has at most 4 significant bits (so it is exact in fp16,
    # bf16 and e4m3)
    for v in pos:
        m, e = math.frexp(v)
        assert (m * 16) == int(m * 16)
        assert float(np.float16(v)) == v
    # exhaustive search over the 4-significant-bit values within 15% of each of
    # Max's levels (vectorised over all increasing combinations): the
    # codebook is the least-MSE choice
    def grid_near(v):
        out = []
        for e in range(-6, 4):
            for mant in range(8, 16):
                x = mant * 2.0 ** (e - 3)
                if abs(x - v) <= 0.15 * v + 0.02:
                    out.append(x)
        return sorted(set(out))
    cands = [grid_near(v) for v in g["positive_output_levels"]]
    combos = np.array(list(itertools.product(*cands)))
    combos = combos[np.all(np.diff(combos, axis=1) > 0, axis=1)]
    full = np.concatenate([-combos[:, ::-1], combos], axis=1)          # (N, 16)
    t = (full[:, :-1] + full[:, 1:]) / 2
    a_ = np.concatenate([np.full((len(t), 1), -np.inf), t], axis=1)
    b_ = np.concatenate([t, np.full((len(t), 1), np.inf)], axis=1)
    m0 = norm.cdf(b_) - norm.cdf(a_)
    m1 = norm.pdf(a_) - norm.pdf(b_)
    m2 = m0 + np.where(np.isinf(a_), 0, a_) * norm.pdf(a_) - np.where(np.isinf(b_), 0, b_) * norm.pdf(b_)
    mse_all = np.sum(m2 - 2 * full * m1 + full * full * m0, axis=1)
    assert len(combos) > 1000
    assert tuple(pos) == tuple(combos[np.argmin(mse_all)])
    assert abs(mse_all.min() - _gauss_mse(o.CODEBOOK)) < 1e-15
    # it costs less than 3% over the unconstrained Lloyd-Max quantiser
    assert g["mse"] < _gauss_mse(o.CODEBOOK) < 1.03 * g["mse"]


# ---------------------------------------------------------------- code rule
def _levels_toward_zero_first():
    """Levels ordered (+0.125, -0.125, +0.375, -0.375, ...): argmin over this
    order breaks distance ties toward the smaller magnitude, and at 0 toward +."""
    lv = []
    for m in o.MAGNITUDES:
        lv += [m, -m]
    return np.array(lv)


def test_code_is_nearest_level_ties_toward_zero():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((300, 128)) * rng.uniform(0.01, 100, size=(300, 1))
    _, codes, d_bits = o.quantize_blocks(x.astype(np.float32))
    u = o.rotate(x.astype(np.float32).astype(np.float64), o.sign_vector(0))
    d = o.half_bits_to_float(d_bits)
    lv = _levels_toward_zero_first()
    nearest = lv[np.argmin(np.abs(u[..., None] - d[:, None, None] * lv), axis=-1)]
    assert np.array_equal(o.CODE_VALUES[codes] * d[:, None], nearest * d[:, None])
    # the code's sign bit is the sign of u; its magnitude rank is the level's
    assert np.array_equal(codes >= 8, u < 0)
    assert np.array_equal(o.MAGNITUDES[codes & 7], np.abs(nearest))


def test_code_exact_ties_and_zero():
    # |u| exactly on the midpoint between magnitudes m and m+1 takes m, for
    # either sign; u = 0 takes +0.125 (code 0).
    d = 0.5
    for k, t in enumerate(o.MAG_THRESHOLDS):
        u = d * t
        assert int((d * o.MAG_THRESHOLDS < abs(u)).sum()) == k
        assert int((d * o.MAG_THRESHOLDS < abs(-u)).sum()) == k
    packed, codes, d_bits = o.quantize_blocks(np.zeros((1, 128)))
    assert np.all(codes == 0) and np.all(packed == 0)
    assert np.array_equal(o.CODE_VALUES, np.concatenate([o.MAGNITUDES, -o.MAGNITUDES]))
    assert np.array_equal(np.sort(o.CODE_VALUES), o.CODEBOOK)
    assert np.array_equal(o.MAG_THRESHOLDS, o.THRESHOLDS[8:])


# ---------------------------------------------------------------- known blocks
@pytest.mark.parametrize("blk", _gold("known_blocks.json")["blocks"], ids=lambda b: b["name"])
def test_known_answer_blocks(blk):
    x = np.zeros(128, np.float32)
    if blk["input"]["kind"] == "unit":
        x[blk["input"]["index"]] = blk["input"]["value"]
    packed, _, _ = o.quantize_blocks(x, seed=blk["seed"])
    assert packed.tobytes().hex() == blk["hex"]
    assert bytes(so.quantize_block(x, seed=blk["seed"])).hex() == blk["hex"]


# ---------------------------------------------------------------- vector vs scalar twin
def test_vectorised_matches_scalar_twin():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal((40, 128)),
        rng.standard_t(3, size=(20, 128)) * 30,
        rng.standard_normal((10, 128)) * 1e-6,
        np.eye(128)[:5] * 7.0,
    ]).astype(np.float32)
    x[3, 17] = 4000.0                           # outlier
    for seed in (0, 7, 123456789):
        packed, _, _ = o.quantize_blocks(x, seed=seed)
        for r in range(len(x)):
            assert list(packed[r]) == so.quantize_block(x[r], seed=seed), (seed, r)
        xd = o.dequantize_blocks(packed[:6], seed=seed)
        for r in range(6):
            np.testing.assert_allclose(xd[r], so.dequantize_block(list(packed[r]), seed), atol=1e-13)


def test_input_dtypes_are_exact():
    rng = np.random.default_rng(6)
    x32 = rng.standard_normal((8, 128)).astype(np.float32)
    x16 = x32.astype(np.float16)
    p16, _, _ = o.quantize_blocks(x16)
    p32, _, _ = o.quantize_blocks(x16.astype(np.float32))
    assert np.array_equal(p16, p32)


def test_saturation_and_tiny_blocks():
    x = np.full((1, 128), 1e30, np.float32)     # RMS far above 65504
    packed, idx, d = o.quantize_blocks(x)
    assert int(d[0]) == 0x7BFF
    y = np.full((1, 128), 1e-30, np.float32)    # RMS below 2^-25 -> d = 0
    packed, idx, d = o.quantize_blocks(y)
    assert int(d[0]) == 0
    assert np.all(o.dequantize_blocks(packed) == 0)


# ---------------------------------------------------------------- round trip
def test_roundtrip_error_matches_codebook_mse():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((20000, 128))
    packed, _, _ = o.quantize_blocks(x.astype(np.float32))
    xh = o.dequantize_blocks(packed)
    x32 = x.astype(np.float32).astype(np.float64)
    rel = np.mean(np.sum((xh - x32) ** 2, axis=1) / np.sum(x32 ** 2, axis=1))
    # per-coordinate Gaussian MSE 0.00972 for this codebook; block RMS scaling
    # brings it to about 0.0096.
    assert 0.0090 < rel < 0.0100


def test_unpack_inverts_pack():
    rng = np.random.default_rng(7)
    packed, idx, d_bits = o.quantize_blocks(rng.standard_normal((64, 128)).astype(np.float32))
    idx2, d = o.unpack_blocks(packed)
    assert np.array_equal(idx, idx2)
    assert np.array_equal(d, o.half_bits_to_float(d_bits))
    # dequantised rotated values are exactly d * level
    y = o.dequantize_rotated(packed)
    for r in range(3):
        for i in range(128):
            assert y[r, i] == float(Fraction(d[r]) * Fraction(o.CODE_VALUES[idx[r, i]]))


def _nearest_binary16_bruteforce(x):
    """Nearest finite binary16 by search over every bit pattern (exact
    rationals); ties to the even pattern; |x| >= 65520 overflows to inf."""
    from fractions import Fraction
    import bisect
    vals = sorted({Fraction(float(np.uint16(b).view(np.float16))): None
                   for b in range(0x7C00)}.keys())            # +0 .. 65504
    out = []
    for xv in x:
        f = Fraction(float(xv))
        a = abs(f)
        if a >= 65520:
            out.append(np.float16(np.inf) if f > 0 else np.float16(-np.inf))
            continue
        i = bisect.bisect_left(vals, a)
        if i == len(vals):            # (65504, 65520): below the overflow midpoint
            r = vals[-1]
        elif vals[i] == a:
            r = vals[i]
        else:
            lo, hi = vals[i - 1], vals[i]
            if a - lo < hi - a:
                r = lo
            elif hi - a < a - lo:
                r = hi
            else:   # tie: the even bit pattern
                r = lo if (np.float16(float(lo)).view(np.uint16) & 1) == 0 else hi
        out.append(-np.float16(float(r)) if np.signbit(xv) else np.float16(float(r)))
    return np.array(out, dtype=np.float16)


def test_f16_rows_round_to_nearest_even_against_bruteforce():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(300).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 5, 300),
        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24, 2 ** -25, 3 * 2 ** -26,
                  65504.0, 65519.0, 65520.0, -65520.0, 1e6, -0.0, 0.0], dtype=np.float32),
    ])
    with np.errstate(over="ignore"):
        got = o.f16_rows(x)
    ref = _nearest_binary16_bruteforce(x)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    # exact halfway cases go to the even pattern: 1 + 2^-11 -> 1.0, 1 + 3*2^-11 -> 1 + 2^-9
    assert o.f16_rows(np.float32(1 + 2 ** -11)) == np.float16(1.0)
    assert o.f16_rows(np.float32(1 + 3 * 2 ** -11)) == np.float16(1 + 2 ** -9)
    assert np.array_equal(o.dequantize_f16(got[:5]), got[:5].astype(np.float64))
