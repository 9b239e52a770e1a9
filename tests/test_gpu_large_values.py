"""Peaky attention over large V values, at the bare bound (fp32 output).

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "Od czego zacząłem": flash attention straight on the TBQ4 blocks.  The
kernels fold the V block scale into the softmax weight (P~ = p d^V) before the
PV product; if P~ were a single fp16 value, its rounding (relative 2^-11 per
weight, the same for the whole 128-value row) would move the output by up to
2^-11 of the few dominant V rows -- about 1e-2 when one V channel is x36 and a
handful of keys carry the weight.  These cases put exactly that in front of
decode, verify and prefill: a V channel scaled x36, two to a few thousand
cached tokens, keys scaled up to x6 so that few keys dominate, fp32 output,
max-abs 2e-3 and relative L2 1e-3 with no allowance.
"""

import math

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)


def _inputs(seed, B, T, H, G, n_q, kmag):
    """fp32 k, v [B][T][H][128] with one V channel x36 per (sequence, head),
    keys x kmag; q [B][n_q][H*G][128]."""
    rng = np.random.default_rng([7, seed])
    k = rng.standard_normal((B, T, H, 128)) * kmag
    v = rng.standard_normal((B, T, H, 128))
    for b in range(B):
        for h in range(H):
            v[b, :, h, rng.integers(128)] *= 36.0
    q = rng.standard_normal((B, n_q, H * G, 128))
    return k.astype(np.float32), v.astype(np.float32), q.astype(np.float32)


def _cache(k, v, cap, seed=0):
    B, T, H, _ = k.shape
    cache = tb.KVCache(B, H, cap, sign_seed=seed)
    tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0]
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kc)
    assert np.array_equal(cache.v[:, :, :T].cpu().numpy(), vc)
    return cache, kc, vc


CASES = [(s, T, kmag) for s, (T, kmag) in enumerate(
    [(2, 1.0), (3, 1.0), (3, 3.0), (5, 6.0), (7, 3.0), (17, 6.0), (64, 6.0), (1000, 6.0),
     (4000, 3.0)])]


@pytest.mark.parametrize("seed,T,kmag", CASES)
def test_decode(seed, T, kmag):
    k, v, q = _inputs(seed, 2, T, 2, 8, 1, kmag)
    cap = ((T + 7) // 8) * 8
    cache, kc, vc = _cache(k, v, cap)
    ref = o.attn_decode_ref(q[:, 0], kc, vc, T, SCALE)
    for P in sorted({1, 2, max(1, T // 200)}):
        out = tb.attn_decode(cache, torch.from_numpy(q[:, 0]).cuda(), T, SCALE, n_splits=P,
                             out_dtype=torch.float32).cpu().numpy()
        check_attn(out, ref, False, f"decode T={T} kmag={kmag} P={P}")


@pytest.mark.parametrize("n_q", [1, 2, 3, 4])
@pytest.mark.parametrize("seed,T,kmag", CASES[1:7])
def test_verify(seed, T, kmag, n_q):
    k, v, q = _inputs(100 + seed, 2, T + n_q, 2, 8, n_q, kmag)
    cap = ((T + n_q + 7) // 8) * 8
    cache, kc, vc = _cache(k, v, cap)
    ref = o.attn_prefill_ref(q, kc, vc, T, SCALE)
    out = tb.attn_verify(cache, torch.from_numpy(q).cuda(), T, SCALE,
                         out_dtype=torch.float32).cpu().numpy()
    check_attn(out, ref, False, f"verify T={T} n_q={n_q} kmag={kmag}")


@pytest.mark.parametrize("seed,n_past,n_q,kmag", [
    (0, 0, 3, 1.0), (1, 1, 4, 3.0), (2, 4, 40, 6.0), (3, 60, 80, 6.0), (4, 500, 100, 3.0),
    (5, 2000, 64, 6.0)])
def test_prefill(seed, n_past, n_q, kmag):
    k, v, q = _inputs(200 + seed, 1, n_past + n_q, 2, 8, n_q, kmag)
    cap = ((n_past + n_q + 7) // 8) * 8
    cache, kc, vc = _cache(k, v, cap)
    ref = o.attn_prefill_ref(q, kc, vc, n_past, SCALE)
    out = tb.attn_prefill_chunk(cache, torch.from_numpy(q).cuda(), n_past, SCALE,
                                out_dtype=torch.float32).cpu().numpy()
    check_attn(out, ref, False, f"prefill n_past={n_past} n_q={n_q} kmag={kmag}")
