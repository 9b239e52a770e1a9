"""Seeded random shapes for decode, prefill and verify against the fp64 oracle.

Each case draws batch, KV heads, group size, lengths (ragged against the
32-token tile and the 64-key prefill tile, down to a single cached token),
split count, sign seed, softmax scale and input / output dtypes from its own
seed.  K rows are Student-t with per-channel scales and one x12 outlier
channel; V rows are Gaussian with per-channel scales, bounded by 4.  The
kernels round P~ = p d^V to fp16 (unit roundoff 2^-11), so when a few keys
dominate the softmax the output error is up to 2^-11 of the V values they
carry: with |v| <= 4 that stays inside the absolute bar for any attention
pattern and any length.  The packed caches must match the oracle's bytes;
outputs must meet the attention bar (max-abs 2e-3 and relative L2 1e-3, plus
half an fp16 ulp for fp16 output).
"""

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu


def _k_rows(rng, B, T, H):
    x = rng.standard_t(5, size=(B, T, H, 128)) * rng.uniform(0.5, 3.0, size=(1, 1, H, 128))
    x[..., int(rng.integers(0, 128))] *= 12.0
    return x.astype(np.float32)


def _v_rows(rng, B, T, H):
    x = rng.standard_normal((B, T, H, 128)) * rng.uniform(0.5, 1.5, size=(1, 1, H, 128))
    return x.astype(np.float32)


def _cache(rng, B, H, T, cap, seed):
    k, v = _k_rows(rng, B, T, H), _v_rows(rng, B, T, H)
    cache = tb.KVCache(B, H, cap, sign_seed=seed)
    for t0 in range(0, T, 1000):   # several appends, ragged against the tiles
        t1 = min(T, t0 + 1000)
        tb.quantize_append(cache, torch.from_numpy(np.ascontiguousarray(k[:, t0:t1])).cuda(),
                           torch.from_numpy(np.ascontiguousarray(v[:, t0:t1])).cuda(), t0)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0]
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kc), "K bytes"
    assert np.array_equal(cache.v[:, :, :T].cpu().numpy(), vc), "V bytes"
    return cache, kc, vc


def _cap(rng, n):
    return ((n + int(rng.integers(0, 90)) + 7) // 8) * 8


@pytest.mark.parametrize("case", range(12))
def test_decode_random(case):
    rng = np.random.default_rng(5000 + case)
    B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2, 4]))
    G = int(rng.integers(1, 9))
    n_ctx = int(rng.integers(1, 2600))
    cap = _cap(rng, n_ctx)
    P = int(rng.choice([0, 1, 2, 5, 16, 64, 200]))
    seed = int(rng.integers(0, 2 ** 62))
    scale = float(rng.uniform(0.04, 0.2))
    q_dtype = [torch.float32, torch.float16][int(rng.integers(0, 2))]
    out_dtype = [torch.float32, torch.float16][int(rng.integers(0, 2))]
    cache, kc, vc = _cache(rng, B, H, n_ctx, cap, seed)
    q = torch.from_numpy(rng.standard_normal((B, H * G, 128)).astype(np.float32)).to(q_dtype).cuda()
    out = tb.attn_decode(cache, q, n_ctx, scale, n_splits=P, out_dtype=out_dtype)
    ref = o.attn_decode_ref(q.float().cpu().numpy(), kc, vc, n_ctx, scale, seed)
    check_attn(out.float().cpu().numpy(), ref, out_dtype == torch.float16,
               f"decode case {case}: B={B} H={H} G={G} n_ctx={n_ctx} P={P}")


@pytest.mark.parametrize("case", range(8))
def test_prefill_random(case):
    rng = np.random.default_rng(6000 + case)
    B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    n_past, n_q = int(rng.integers(0, 1500)), int(rng.integers(1, 300))
    cap = _cap(rng, n_past + n_q)
    seed = int(rng.integers(0, 2 ** 62))
    scale = float(rng.uniform(0.04, 0.2))
    out_dtype = [torch.float32, torch.float16][int(rng.integers(0, 2))]
    cache, kc, vc = _cache(rng, B, H, n_past + n_q, cap, seed)
    q = torch.from_numpy(rng.standard_normal((B, n_q, H * G, 128)).astype(np.float32)).cuda()
    out = tb.attn_prefill_chunk(cache, q, n_past, scale, out_dtype=out_dtype)
    ref = o.attn_prefill_ref(q.cpu().numpy(), kc, vc, n_past, scale, seed)
    check_attn(out.float().cpu().numpy(), ref, out_dtype == torch.float16,
               f"prefill case {case}: B={B} H={H} G={G} n_past={n_past} n_q={n_q}")


@pytest.mark.parametrize("case", range(8))
def test_verify_random(case):
    rng = np.random.default_rng(7000 + case)
    B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2]))
    G = int(rng.integers(1, 9))
    n_q = int(rng.integers(1, 5))
    n_past = int(rng.integers(0, 2400))
    cap = _cap(rng, n_past + n_q)
    P = int(rng.choice([0, 1, 3, 16, 64]))
    seed = int(rng.integers(0, 2 ** 62))
    scale = float(rng.uniform(0.04, 0.2))
    cache, kc, vc = _cache(rng, B, H, n_past + n_q, cap, seed)
    q = torch.from_numpy(rng.standard_normal((B, n_q, H * G, 128)).astype(np.float32)).cuda()
    out = tb.attn_verify(cache, q, n_past, scale, n_splits=P, out_dtype=torch.float32)
    ref = o.attn_prefill_ref(q.cpu().numpy(), kc, vc, n_past, scale, seed)
    check_attn(out.cpu().numpy(), ref, False,
               f"verify case {case}: B={B} H={H} G={G} n_q={n_q} n_past={n_past} P={P}")
