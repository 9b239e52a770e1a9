"""Pins of the oracle's attention against closed forms and library routines.

Attention: page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Od czego zacząłem" -- flash attention over the
TBQ4 cache, computed in the rotated (Hadamard) domain.  Flash attention
computes exactly softmax attention, so the oracle is that definition.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

from oracle import scalar_oracle as so
from oracle import tbq4_oracle as o
from workloads import WORKLOADS, tiny_inputs


def _cache(rng, B, H, T, scale=1.0, seed=0):
    x = (rng.standard_normal((B, H, T, 128)) * scale).astype(np.float32)
    return o.quantize_blocks(x, seed=seed)[0]


def test_decode_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(10)
    B, Hkv, G, T = 2, 3, 4, 37
    kc, vc = _cache(rng, B, Hkv, T), _cache(rng, B, Hkv, T)
    q = rng.standard_normal((B, Hkv * G, 128))
    scale = 0.3
    got = o.attn_decode_ref(q, kc, vc, T, scale)
    K = torch.from_numpy(o.dequantize_blocks(kc))
    Vt = torch.from_numpy(o.dequantize_blocks(vc))
    want = F.scaled_dot_product_attention(torch.from_numpy(q)[:, :, None], K, Vt,
                                          scale=scale, enable_gqa=True)[:, :, 0]
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_matches_torch_sdpa_lower_right_causal():
    rng = np.random.default_rng(11)
    B, Hkv, G, n_past, n_q = 1, 2, 3, 20, 9
    T = n_past + n_q
    kc, vc = _cache(rng, B, Hkv, T + 5), _cache(rng, B, Hkv, T + 5)
    q = rng.standard_normal((B, n_q, Hkv * G, 128))
    got = o.attn_prefill_ref(q, kc, vc, n_past, 0.2)
    K = torch.from_numpy(o.dequantize_blocks(kc[:, :, :T]))
    Vt = torch.from_numpy(o.dequantize_blocks(vc[:, :, :T]))
    qt = torch.from_numpy(q).transpose(1, 2)
    want = F.scaled_dot_product_attention(qt, K, Vt, attn_mask=causal_lower_right(n_q, T),
                                          scale=0.2, enable_gqa=True).transpose(1, 2)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_rows_equal_decode_at_their_length():
    rng = np.random.default_rng(12)
    n_past, n_q = 15, 6
    kc, vc = _cache(rng, 1, 2, n_past + n_q), _cache(rng, 1, 2, n_past + n_q)
    q = rng.standard_normal((1, n_q, 4, 128))
    pre = o.attn_prefill_ref(q, kc, vc, n_past, 0.1)
    for i in (0, n_q - 1):
        dec = o.attn_decode_ref(q[:, i], kc, vc, n_past + i + 1, 0.1)
        np.testing.assert_allclose(pre[:, i], dec, rtol=1e-13, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(13)
    kc, vc = _cache(rng, 1, 1, 16), _cache(rng, 1, 1, 16)
    V = o.dequantize_blocks(vc[0, 0])
    q = rng.standard_normal((1, 2, 128))
    # one key: o = v_0 exactly
    np.testing.assert_array_equal(o.attn_decode_ref(q, kc, vc, 1, 1.0)[0, 0], V[0])
    # q = 0: uniform weights, o = mean of V
    np.testing.assert_allclose(o.attn_decode_ref(np.zeros((1, 1, 128)), kc, vc, 16, 1.0)[0, 0],
                               V.mean(axis=0), atol=1e-14)
    # all keys equal: mean of V
    keq = np.repeat(kc[:, :, :1], 16, axis=2)
    np.testing.assert_allclose(o.attn_decode_ref(q, keq, vc, 16, 1.0)[0, 1], V.mean(axis=0), atol=1e-14)
    # two keys: logistic weight
    K = o.dequantize_blocks(kc[0, 0])
    s0, s1 = 0.7 * q[0, 0] @ K[0], 0.7 * q[0, 0] @ K[1]
    w = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(o.attn_decode_ref(q[:, :1], kc, vc, 2, 0.7)[0, 0],
                               w * V[0] + (1 - w) * V[1], atol=1e-14)


def test_rotated_domain_equals_unrotated():
    """Scores in the rotated domain equal scores on dequantised keys because
    the rotation is orthogonal; both decode forms agree on the tiny workload."""
    k, v, q, _ = tiny_inputs()
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3))[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3))[0]
    sc = WORKLOADS["tiny"].softmax_scale
    a = o.attn_decode_ref(q, kc, vc, 1024, sc)
    b = o.attn_decode_rotated_ref(q, kc, vc, 1024, sc)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    s = o.sign_vector(0)
    y = o.dequantize_rotated(kc[0, 0, :5])
    qq = q[0, :1].astype(np.float64)
    np.testing.assert_allclose(o.rotate(qq, s) @ y.T, qq @ o.unrotate(y, s).T, rtol=1e-12)


def test_split_merge_is_partition_invariant():
    rng = np.random.default_rng(14)
    n = 1000
    s = rng.standard_normal(n) * 3
    V = rng.standard_normal((n, 128))
    full = o.merge_partials(o.split_partials(s, V, [(0, n)]))
    p = np.exp(s - s.max())
    np.testing.assert_allclose(full, (p / p.sum()) @ V, rtol=1e-13)
    for P in (2, 7, 16, 256):
        edges = np.linspace(0, n, P + 1).astype(int)
        parts = o.split_partials(s, V, [(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a])
        np.testing.assert_allclose(o.merge_partials(parts), full, rtol=1e-13, atol=1e-15)


def test_tiny_workload_scalar_twin():
    """The whole tiny workload (quantise 2 x 1024 blocks, decode 4 heads) through
    the scalar pure-Python twin: identical bytes, attention within 1e-12."""
    k, v, q, ch = tiny_inputs()
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3))[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3))[0]
    for t in range(0, 1024, 97):
        assert list(kc[0, 0, t]) == so.quantize_block(k[0, t, 0])
        assert list(vc[0, 0, t]) == so.quantize_block(v[0, t, 0])
    sc = WORKLOADS["tiny"].softmax_scale
    got = o.attn_decode_ref(q, kc, vc, 1024, sc)
    keys = [so.dequantize_block(list(b)) for b in kc[0, 0]]
    vals = [so.dequantize_block(list(b)) for b in vc[0, 0]]
    for h in range(4):
        want = so.attend(list(q[0, h].astype(np.float64)), keys, vals, sc)
        np.testing.assert_allclose(got[0, h], want, rtol=1e-11, atol=1e-13)
    # the outlier channel is really there
    assert np.abs(k[0, :, 0, ch]).mean() > 10


@pytest.mark.parametrize("G", [1, 4, 8])
def test_gqa_mapping_distinct_heads(G):
    """Query head h reads KV head h // G: make each KV head's values constant
    and distinct, then every query head's output is its KV head's constant."""
    Hkv, T = 3, 5
    vc = np.empty((1, Hkv, T, 66), np.uint8)
    rng = np.random.default_rng(15)
    for g in range(Hkv):
        vc[0, g] = o.quantize_blocks(np.full((T, 128), g + 1.0, np.float32))[0]
    kc = _cache(rng, 1, Hkv, T)
    out = o.attn_decode_ref(rng.standard_normal((1, Hkv * G, 128)), kc, vc, T, 1.0)
    for h in range(Hkv * G):
        want = o.dequantize_blocks(vc[0, h // G, 0])
        np.testing.assert_allclose(out[0, h], want, atol=1e-12)
