"""GPU prefill-chunk attention against the fp64 oracle.

Method: page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Od czego zacząłem" (flash attention straight on
TBQ4 blocks in the rotated domain).  A chunk's query i sits at position
n_past + i and attends keys 0 .. n_past + i; the chunk's own K/V are appended
first.  Bar: max-abs 2e-3 and relative L2 1e-3 (plus half an fp16 ulp of the
reference for fp16 output).
"""

import math

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from workloads import WORKLOADS, kv_rows, kv_tensor, q_prefill
from _util import check_attn

pytestmark = pytest.mark.gpu


def _case(B, Hkv, G, n_past, n_q, cap, scale, seed=0, rng_seed=0, q_dtype=torch.float32,
          out_dtype=torch.float32, kscale=1.0):
    rng = np.random.default_rng(rng_seed)
    T = n_past + n_q
    k = (rng.standard_normal((B, T, Hkv, 128)) * kscale).astype(np.float32)
    v = rng.standard_normal((B, T, Hkv, 128)).astype(np.float32)
    q = rng.standard_normal((B, n_q, Hkv * G, 128)).astype(np.float32)
    cache = tb.KVCache(B, Hkv, cap, sign_seed=seed)
    if n_past:
        tb.quantize_append(cache, torch.from_numpy(k[:, :n_past]).cuda(),
                           torch.from_numpy(v[:, :n_past]).cuda(), 0)
    tb.quantize_append(cache, torch.from_numpy(np.ascontiguousarray(k[:, n_past:])).cuda(),
                       torch.from_numpy(np.ascontiguousarray(v[:, n_past:])).cuda(), n_past)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0]
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kc)
    qt = torch.from_numpy(q).to(q_dtype).cuda()
    out = tb.attn_prefill_chunk(cache, qt, n_past, scale, out_dtype=out_dtype)
    ref = o.attn_prefill_ref(qt.float().cpu().numpy(), kc, vc, n_past, scale, seed)
    return out.float().cpu().numpy(), ref


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32])
def test_group_sizes(G):
    out, ref = _case(1, 2, G, 100, 37, 144, 1 / math.sqrt(128), rng_seed=G)
    check_attn(out, ref, False, f"G={G}")


@pytest.mark.parametrize("n_past,n_q", [(0, 1), (0, 5), (0, 64), (1, 1), (5, 3), (63, 2),
                                        (64, 17), (130, 200), (1000, 19), (2000, 128)])
def test_ragged_chunks(n_past, n_q):
    cap = ((n_past + n_q + 7) // 8) * 8
    out, ref = _case(1, 2, 8, n_past, n_q, cap, 0.1, seed=3, rng_seed=n_past + n_q)
    check_attn(out, ref, False, f"n_past={n_past} n_q={n_q}")


def test_batch_and_fp16_io():
    out, ref = _case(3, 2, 8, 300, 40, 344, 0.08, seed=9, rng_seed=1, q_dtype=torch.float16,
                     out_dtype=torch.float16)
    check_attn(out, ref, True, "batch3 fp16")


def test_peaky_scores():
    out, ref = _case(1, 1, 8, 500, 24, 528, 1 / math.sqrt(128), rng_seed=5, kscale=25.0)
    check_attn(out, ref, False, "peaky")


@pytest.mark.parametrize("scale", [1e-4, 2.0, 30.0])
def test_query_magnitudes(scale):
    """q' is normalised by one power of two per workgroup, which the staged K
    values carry back: tiny queries (the normalisation at its bound, near-
    uniform weights), and large ones (the exponent well inside its range,
    peaky weights) match the oracle like the usual scale."""
    out, ref = _case(1, 2, 8, 300, 40, 344, scale, seed=4, rng_seed=11)
    check_attn(out, ref, False, f"qscale={scale}")


def test_matches_decode_for_single_query():
    """A one-query chunk is a decode step: both paths agree with the oracle."""
    rng = np.random.default_rng(7)
    k = rng.standard_normal((1, 777, 2, 128)).astype(np.float32)
    cache = tb.KVCache(1, 2, 784)
    tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(k).cuda(), 0)
    q = torch.from_numpy(rng.standard_normal((1, 16, 128)).astype(np.float32)).cuda()
    dec = tb.attn_decode(cache, q, 777, 0.1, out_dtype=torch.float32).cpu().numpy()
    pre = tb.attn_prefill_chunk(cache, q[:, None].contiguous(), 776, 0.1,
                                out_dtype=torch.float32).cpu().numpy()[:, 0]
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3))[0]
    ref = o.attn_decode_ref(q.cpu().numpy(), kc, kc, 777, 0.1)
    check_attn(dec, ref, False, "decode")
    check_attn(pre, ref, False, "prefill")


def test_deterministic():
    rng = np.random.default_rng(8)
    k = torch.from_numpy(rng.standard_normal((1, 600, 2, 128)).astype(np.float32)).cuda()
    cache = tb.KVCache(1, 2, 600)
    tb.quantize_append(cache, k, k, 0)
    q = torch.from_numpy(rng.standard_normal((1, 50, 16, 128)).astype(np.float32)).cuda()
    a = tb.attn_prefill_chunk(cache, q, 550, 0.1)
    b = tb.attn_prefill_chunk(cache, q, 550, 0.1)
    assert torch.equal(a, b)


FULL_GROUP = 3        # the KV-head group whose 2048 chunk rows are all checked


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_prefill_workload():
    """Prefill chunk: 2048 queries on 131072 cached tokens, 8 KV / 64 Q heads,
    Q,K,V ~ N(0,1) with outlier channels on K and V; the chunk's K/V are
    appended first.  K and V bytes of every KV head are compared with the
    oracle's; outputs are checked on every row of one head group and on 64
    seeded random rows of every group, with fp16 output and with fp32 output
    at the bare bound; the stress variant whose queries carry two outlier
    channels x15 per head runs on the same rows in fp32-output mode."""
    from _rows import pool_map, prefill_group, random_rows
    w = WORKLOADS["prefill"]
    n_past, n_q = w.n_ctx, w.n_q
    T = n_past + n_q
    H, G = w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    cache = tb.KVCache(1, H, T)
    for t0 in range(0, T, 32768):
        t1 = min(T, t0 + 32768)
        k = kv_tensor(w, 0, 0, t0, t1)
        v = kv_tensor(w, 0, 1, t0, t1)
        tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), t0)
    outs = {}
    for outliers, dtypes in ((False, (torch.float16, torch.float32)), (True, (torch.float32,))):
        qt = torch.from_numpy(q_prefill(w, outliers=outliers)).cuda()
        for od in dtypes:
            outs[(outliers, od)] = tb.attn_prefill_chunk(cache, qt, n_past, w.softmax_scale,
                                                         out_dtype=od).float().cpu().numpy()
        del qt
    kg, vg = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    del cache
    torch.cuda.empty_cache()
    rows = {g: (np.arange(n_q) if g == FULL_GROUP else random_rows([5, g], n_q, 64))
            for g in range(H)}
    jobs = [("prefill", g, rows[g], (False, True)) for g in range(H)]
    for (_, g, r, _), (kc, vc, refs) in zip(jobs, pool_map(prefill_group, jobs)):
        assert np.array_equal(kg[0, g], kc), f"K bytes g={g}"
        assert np.array_equal(vg[0, g], vc), f"V bytes g={g}"
        for (outliers, od), out in outs.items():
            check_attn(out[0, r, g * G:(g + 1) * G], refs[outliers], od == torch.float16,
                       f"prefill g={g} q outliers={outliers} {od}")


def test_unused_slots_with_nan_scales_do_not_leak():
    """Keys at or past n_past + n_q may hold anything (0xFF = NaN scales)."""
    rng = np.random.default_rng(41)
    n_past, n_q = 100, 37
    T = n_past + n_q
    k = rng.standard_normal((1, T, 2, 128)).astype(np.float32)
    v = rng.standard_normal((1, T, 2, 128)).astype(np.float32)
    q = rng.standard_normal((1, n_q, 16, 128)).astype(np.float32)
    cache = tb.KVCache(1, 2, 256)
    cache.k.fill_(0xFF)
    cache.v.fill_(0xFF)
    tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3))[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3))[0]
    out = tb.attn_prefill_chunk(cache, torch.from_numpy(q).cuda(), n_past, 0.1,
                                out_dtype=torch.float32)
    ref = o.attn_prefill_ref(q, kc, vc, n_past, 0.1, 0)
    check_attn(out.cpu().numpy(), ref, False, "nan tail prefill")


def test_bf16_queries():
    out, ref = _case(2, 2, 8, 300, 70, 376, 1 / math.sqrt(128), seed=4, rng_seed=11,
                     q_dtype=torch.bfloat16, out_dtype=torch.float16)
    check_attn(out, ref, True, "bf16 q")
