"""GPU multi-query verify attention against the fp64 oracle.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq": the
production decode verifies the current token plus up to three drafted ones
(--spec-type mtp --spec-draft-n-max 3); section "Od czego zacząłem" gives the
attention (flash attention on TBQ4 blocks in the rotated domain).  Query i
sits at position n_past + i and attends slots 0 .. n_past + i: the oracle is
the prefill-chunk definition at n_q <= 4.  Bar: max-abs 2e-3 and relative L2
1e-3 (plus half an fp16 ulp of the reference for fp16 output).
"""

import math

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from workloads import WORKLOADS, kv_rows, kv_tensor
from _util import check_attn, rising_scores_inputs

pytestmark = pytest.mark.gpu


def _case(B, Hkv, G, n_past, n_q, cap, scale, P=0, seed=0, rng_seed=0, q_dtype=torch.float32,
          out_dtype=torch.float32, kscale=1.0, junk_tail=False):
    rng = np.random.default_rng(rng_seed)
    T = n_past + n_q
    k = (rng.standard_normal((B, T, Hkv, 128)) * kscale).astype(np.float32)
    v = rng.standard_normal((B, T, Hkv, 128)).astype(np.float32)
    q = rng.standard_normal((B, n_q, Hkv * G, 128)).astype(np.float32)
    cache = tb.KVCache(B, Hkv, cap, sign_seed=seed)
    if junk_tail:   # slots past the drafted tokens hold NaN scales and random codes
        cache.k.fill_(0xFF)
        cache.v.fill_(0xFF)
    tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0]
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kc)
    qt = torch.from_numpy(q).to(q_dtype).cuda()
    out = tb.attn_verify(cache, qt, n_past, scale, n_splits=P, out_dtype=out_dtype)
    ref = o.attn_prefill_ref(qt.float().cpu().numpy(), kc, vc, n_past, scale, seed)
    return out.float().cpu().numpy(), ref


@pytest.mark.parametrize("n_q", [1, 2, 3, 4])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_queries_and_groups(n_q, G):
    out, ref = _case(2, 2, G, 700, n_q, 712, 1 / math.sqrt(128), P=5, rng_seed=10 * n_q + G)
    check_attn(out, ref, False, f"n_q={n_q} G={G}")


@pytest.mark.parametrize("n_past,n_q", [(0, 1), (0, 4), (1, 3), (28, 4), (29, 3), (31, 1),
                                        (32, 2), (63, 4), (1000, 4)])
def test_tile_boundaries(n_past, n_q):
    """Draft tokens straddling 32-slot tiles; a cache whose unused slots
    hold NaN scales must not leak into the result."""
    cap = ((n_past + n_q + 7) // 8) * 8 + 32
    out, ref = _case(1, 2, 8, n_past, n_q, cap, 0.1, P=3, seed=2, rng_seed=n_past + 7 * n_q,
                     junk_tail=True)
    check_attn(out, ref, False, f"n_past={n_past} n_q={n_q}")


@pytest.mark.parametrize("P", [1, 2, 16, 64, 0])
def test_split_counts(P):
    out, ref = _case(1, 1, 8, 4000, 4, 4008, 0.09, P=P, rng_seed=P)
    check_attn(out, ref, False, f"P={P}")


def test_fp16_queries_fp16_output_and_peaky_scores():
    out, ref = _case(1, 2, 8, 1500, 4, 1512, 1 / math.sqrt(128), P=7, q_dtype=torch.float16,
                     out_dtype=torch.float16, rng_seed=3)
    check_attn(out, ref, True, "fp16 io")
    out, ref = _case(1, 1, 8, 2000, 3, 2008, 1 / math.sqrt(128), P=8, kscale=30.0, rng_seed=4)
    check_attn(out, ref, False, "peaky")


def test_single_query_matches_decode():
    """n_q = 1 at n_past = T - 1 is a decode over T slots."""
    rng = np.random.default_rng(5)
    k = torch.from_numpy(rng.standard_normal((2, 999, 2, 128)).astype(np.float32)).cuda()
    cache = tb.KVCache(2, 2, 1000)
    tb.quantize_append(cache, k, k, 0)
    q = torch.from_numpy(rng.standard_normal((2, 16, 128)).astype(np.float32)).cuda()
    a = tb.attn_decode(cache, q, 999, 0.1, n_splits=4, out_dtype=torch.float32)
    b = tb.attn_verify(cache, q[:, None].contiguous(), 998, 0.1, n_splits=4,
                       out_dtype=torch.float32)[:, 0]
    np.testing.assert_allclose(a.cpu().numpy(), b.cpu().numpy(), atol=2e-4)


@pytest.mark.slow
def test_decode128k_verify_sampled():
    """Verify of 4 queries at the 128K decode shape (batch 4, 8 / 64 heads):
    two (sequence, KV head) rows re-quantised by the oracle and checked."""
    w = WORKLOADS["decode128k"]
    T = w.n_ctx
    n_q = 4
    cache = tb.KVCache(w.batch, w.n_kv_heads, T)
    for t0 in range(0, T, 32768):
        k = kv_tensor(w, 0, 0, t0, t0 + 32768)
        v = kv_tensor(w, 0, 1, t0, t0 + 32768)
        tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), t0)
    rng = np.random.default_rng([0, 2, 77])
    q = rng.standard_normal((w.batch, n_q, w.n_q_heads, 128)).astype(np.float32)
    n_past = T - n_q
    out = tb.attn_verify(cache, torch.from_numpy(q).cuda(), n_past, w.softmax_scale).float().cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    for (b, g) in ((1, 2), (3, 7)):
        kc = o.quantize_blocks(kv_rows(w, 0, 0, b, g, 0, T))[0]
        vc = o.quantize_blocks(kv_rows(w, 0, 1, b, g, 0, T))[0]
        Kh, Vh = o.dequantize_blocks(kc), o.dequantize_blocks(vc)
        for i in range(n_q):
            n = n_past + i + 1
            ref = o.attn_decode_rows_ref(q[b, i, g * G:(g + 1) * G], Kh[:n], Vh[:n], w.softmax_scale)
            check_attn(out[b, i, g * G:(g + 1) * G], ref, True, f"128k verify b={b} g={g} i={i}")


@pytest.mark.parametrize("vmag", [1.0, 300.0, 5000.0])
def test_rising_scores_and_large_v_scales(vmag):
    """As the decode test of the same name, for 4 queries per sequence: the
    lagged reference maximum per column group, exact maxima in tiles with V
    scales above 256; compared after dividing by vmag."""
    rng = np.random.default_rng(50 + int(vmag))
    B, H, G, n_q, n_past = 1, 2, 8, 4, 4092
    T = n_past + n_q
    q, k, v = rising_scores_inputs(rng, B, T, H, G, n_q, vmag)
    cache = tb.KVCache(B, H, T, sign_seed=3)
    tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3), 3)[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3), 3)[0]
    out = tb.attn_verify(cache, torch.from_numpy(q).cuda(), n_past, 1 / math.sqrt(128), n_splits=2,
                         out_dtype=torch.float32).cpu().numpy()
    ref = o.attn_prefill_ref(q, kc, vc, n_past, 1 / math.sqrt(128), 3)
    check_attn(out / vmag, ref / vmag, False, f"vmag={vmag}")
    if vmag <= 300.0:   # and at the bare absolute bound while |V| stays in the hundreds
        check_attn(out, ref, False, f"bare bound vmag={vmag}")


def test_bf16_queries():
    out, ref = _case(2, 2, 8, 900, 4, 912, 1 / math.sqrt(128), P=3, q_dtype=torch.bfloat16,
                     rng_seed=9)
    check_attn(out, ref, False, "bf16 q")
