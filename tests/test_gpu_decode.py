"""GPU split-K decode attention against the fp64 oracle.

Method: page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Od czego zacząłem" (flash attention straight on
TBQ4 blocks, dequantised in the inner loop, in the rotated domain).  Bar:
packed caches byte-identical to the oracle's; outputs within max-abs 2e-3 and
relative L2 1e-3 (plus half an fp16 ulp of the reference for fp16 output).
"""

import math

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from workloads import WORKLOADS, kv_rows, kv_tensor, q_decode, tiny_inputs
from _util import check_attn, rising_scores_inputs

pytestmark = pytest.mark.gpu


def _fill(cache, k, v, chunk=16384):
    """Append host fp32 [B][T][H][128] K/V into the cache in chunks."""
    T = k.shape[1]
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        tb.quantize_append(cache, torch.from_numpy(np.ascontiguousarray(k[:, t0:t1])).cuda(),
                           torch.from_numpy(np.ascontiguousarray(v[:, t0:t1])).cuda(), t0)


def _oracle_cache(k, v, seed=0):
    # [B][T][H][128] -> [B][H][T][66]
    return (o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0],
            o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0])


def _run_small(B, Hkv, G, T, cap, n_ctx, scale, seed, P, q_dtype=torch.float32,
               out_dtype=torch.float16, rng_seed=0, kscale=1.0):
    rng = np.random.default_rng(rng_seed)
    k = (rng.standard_normal((B, T, Hkv, 128)) * kscale).astype(np.float32)
    v = rng.standard_normal((B, T, Hkv, 128)).astype(np.float32)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    cache = tb.KVCache(B, Hkv, cap, sign_seed=seed)
    _fill(cache, k, v)
    kc, vc = _oracle_cache(k, v, seed)
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kc)
    assert np.array_equal(cache.v[:, :, :T].cpu().numpy(), vc)
    qt = torch.from_numpy(q).to(q_dtype).cuda()
    out = tb.attn_decode(cache, qt, n_ctx, scale, n_splits=P, out_dtype=out_dtype)
    ref = o.attn_decode_ref(qt.float().cpu().numpy(), kc, vc, n_ctx, scale, seed)
    return out.float().cpu().numpy(), ref


def test_tiny_workload_full():
    """Tiny decode: batch 1, 1 KV / 4 Q heads, 1024 tokens, one key channel x20."""
    w = WORKLOADS["tiny"]
    k, v, q, _ = tiny_inputs()
    cache = tb.KVCache(1, 1, 1024)
    _fill(cache, k, v)
    kc, vc = _oracle_cache(k, v)
    assert np.array_equal(cache.k.cpu().numpy(), kc)
    assert np.array_equal(cache.v.cpu().numpy(), vc)
    ref = o.attn_decode_ref(q, kc, vc, 1024, w.softmax_scale)
    for P in (0, 1, 2, 4, 16):
        for od in (torch.float16, torch.float32):
            out = tb.attn_decode(cache, torch.from_numpy(q).cuda(), 1024, w.softmax_scale,
                                 n_splits=P, out_dtype=od)
            check_attn(out.float().cpu().numpy(), ref, od == torch.float16, f"tiny P={P} {od}")


@pytest.mark.parametrize("n_ctx", [1, 2, 7, 63, 64, 65, 129, 200, 1000])
def test_ragged_lengths(n_ctx):
    cap = ((n_ctx + 7) // 8) * 8 + 8
    out, ref = _run_small(1, 2, 8, n_ctx, cap, n_ctx, 1 / math.sqrt(128), seed=3, P=0, rng_seed=n_ctx)
    check_attn(out, ref, True, f"n_ctx={n_ctx}")


@pytest.mark.parametrize("G", [1, 2, 3, 5, 8])
def test_group_sizes(G):
    out, ref = _run_small(2, 3, G, 300, 304, 300, 0.2, seed=11, P=3, rng_seed=G)
    check_attn(out, ref, True, f"G={G}")


def test_n_ctx_shorter_than_filled():
    out, ref = _run_small(2, 2, 4, 512, 512, 333, 0.1, seed=0, P=5)
    check_attn(out, ref, True, "n_ctx < filled")


def test_fp16_queries_and_fp32_output():
    out, ref = _run_small(1, 2, 8, 777, 784, 777, 0.09, seed=1, P=4, q_dtype=torch.float16,
                          out_dtype=torch.float32)
    check_attn(out, ref, False, "fp16 q")


def test_large_scores_peaky_softmax():
    # keys x30 -> very peaky softmax; the online max must stay exact
    out, ref = _run_small(1, 1, 8, 2048, 2048, 2048, 1 / math.sqrt(128), seed=2, P=8,
                          out_dtype=torch.float32, kscale=30.0)
    check_attn(out, ref, False, "peaky")


@pytest.mark.parametrize("P", [1, 3, 16, 64, 256, 1024])
def test_split_counts_agree(P):
    out, ref = _run_small(1, 1, 8, 4096, 4096, 4096, 0.1, seed=4, P=P, out_dtype=torch.float32)
    check_attn(out, ref, False, f"P={P}")


@pytest.mark.parametrize("n_ctx,P", [(4113, 64), (4113, 65), (4113, 13), (4096, 64), (4096, 65),
                                      (4096, 43), (90, 64), (33, 3)])
def test_split_ranges(n_ctx, P):
    """Batch 2, 8 KV heads, about one streaming wavefront per SIMD: split
    ranges of odd and even tile counts, a ragged last tile, splits with a
    single tile and empty splits, in fp32 output against the oracle."""
    out, ref = _run_small(2, 8, 2, 4113, 4128, n_ctx, 0.1, seed=6, P=P, out_dtype=torch.float32,
                          rng_seed=n_ctx + P)
    check_attn(out, ref, False, f"n_ctx={n_ctx} P={P}")


def test_deterministic():
    rng = np.random.default_rng(9)
    k = rng.standard_normal((1, 3000, 2, 128)).astype(np.float32)
    cache = tb.KVCache(1, 2, 3000)
    _fill(cache, k, k)
    q = torch.from_numpy(rng.standard_normal((1, 16, 128)).astype(np.float32)).cuda()
    a = tb.attn_decode(cache, q, 3000, 0.1, n_splits=7)
    b = tb.attn_decode(cache, q, 3000, 0.1, n_splits=7)
    assert torch.equal(a, b)


def test_decode16k_workload_full():
    """Decode at 16384: batch 1, 8 KV / 64 Q heads, 2 outlier channels x15,
    Q ~ N(0,1)/sqrt(128) with scale 1.0 (and again with scale 1/sqrt(128))."""
    w = WORKLOADS["decode16k"]
    T = w.n_ctx
    k = kv_tensor(w, 0, 0, 0, T)
    v = kv_tensor(w, 0, 1, 0, T)
    cache = tb.KVCache(1, 8, T)
    _fill(cache, k, v)
    kc, vc = _oracle_cache(k, v)
    assert np.array_equal(cache.k.cpu().numpy(), kc)
    assert np.array_equal(cache.v.cpu().numpy(), vc)
    q = q_decode(w)
    for scale in (w.softmax_scale, 1 / math.sqrt(128)):
        ref = o.attn_decode_ref(q, kc, vc, T, scale)
        for P in (0, 16, 64):
            for od in (torch.float16, torch.float32):
                out = tb.attn_decode(cache, torch.from_numpy(q).cuda(), T, scale, n_splits=P,
                                     out_dtype=od)
                check_attn(out.float().cpu().numpy(), ref, od == torch.float16,
                           f"16k scale={scale} P={P} {od}")
        # the decode step (bench.py's): the last token appended again (same
        # bytes) and attended in one call
        for P in (0, 64):
            for od in (torch.float16, torch.float32):
                out = tb.decode_step(cache, torch.from_numpy(k[:, T - 1:].copy()).cuda(),
                                     torch.from_numpy(v[:, T - 1:].copy()).cuda(),
                                     torch.from_numpy(q).cuda(), T - 1, scale, n_splits=P,
                                     out_dtype=od)
                check_attn(out.float().cpu().numpy(), ref, od == torch.float16,
                           f"16k decode step scale={scale} P={P} {od}")
    assert np.array_equal(cache.k.cpu().numpy(), kc)
    assert np.array_equal(cache.v.cpu().numpy(), vc)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decode128k_workload_full():
    """Decode at 131072 and at 98304 slots, batch 4, Student-t KV with channel
    scales (the decode96k rows are the first 98304 of the same recipe): the
    whole cache is filled on the GPU; every (sequence, KV head) row is
    re-quantised by the oracle in worker processes (all appended bytes
    compared) and every output of every query head is checked, for split
    counts 16 .. 256 and the automatic one, with fp16 output and with fp32
    output at the bare bound; and the decode step (the last token appended
    again and attended in one call, bench.py's step)."""
    from _rows import decode_row, pool_map
    w = WORKLOADS["decode128k"]
    T = w.n_ctx
    T96 = WORKLOADS["decode96k"].n_ctx
    B, H, G = w.batch, w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    cache = tb.KVCache(B, H, T)
    for t0 in range(0, T, 32768):
        t1 = t0 + 32768
        k = kv_tensor(w, 0, 0, t0, t1)
        v = kv_tensor(w, 0, 1, t0, t1)
        tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), t0)
    q = q_decode(w)
    qt = torch.from_numpy(q).cuda()
    splits = (0, 16, 32, 64, 128, 256)
    outs = {(n, P, od): tb.attn_decode(cache, qt, n, w.softmax_scale, n_splits=P,
                                       out_dtype=od).float().cpu().numpy()
            for n in (T96, T) for P in splits for od in (torch.float16, torch.float32)}
    # the decode step as bench.py times it: the last token appended again
    # (the same row, so the same bytes) and attended in one call
    k_last = torch.from_numpy(kv_tensor(w, 0, 0, T - 1, T)).cuda()
    v_last = torch.from_numpy(kv_tensor(w, 0, 1, T - 1, T)).cuda()
    steps = {(P, od): tb.decode_step(cache, k_last, v_last, qt, T - 1, w.softmax_scale,
                                     n_splits=P, out_dtype=od).float().cpu().numpy()
             for P in (0, 64, 256) for od in (torch.float16, torch.float32)}
    kg, vg = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    del cache
    torch.cuda.empty_cache()
    jobs = [("decode128k", 0, b, g, T,
             [(n, q[b, g * G:(g + 1) * G], n, w.softmax_scale) for n in (T96, T)])
            for b in range(B) for g in range(H)]
    refs = {}
    for (_, _, b, g, _, _), (kc, vc, r) in zip(jobs, pool_map(decode_row, jobs)):
        assert np.array_equal(kg[b, g], kc), f"K bytes b={b} g={g}"
        assert np.array_equal(vg[b, g], vc), f"V bytes b={b} g={g}"
        for n in (T96, T):
            refs.setdefault(n, np.empty((B, w.n_q_heads, 128)))[b, g * G:(g + 1) * G] = r[n]
    for (n, P, od), out in outs.items():
        check_attn(out, refs[n], od == torch.float16, f"n={n} P={P} {od}")
    for (P, od), out in steps.items():
        check_attn(out, refs[T], od == torch.float16, f"decode step P={P} {od}")


def test_two_phase_equals_one_call():
    rng = np.random.default_rng(21)
    k = rng.standard_normal((2, 1500, 2, 128)).astype(np.float32)
    cache = tb.KVCache(2, 2, 1504, sign_seed=4)
    _fill(cache, k, k)
    q = torch.from_numpy(rng.standard_normal((2, 16, 128)).astype(np.float32)).cuda()
    one = tb.attn_decode(cache, q, 1500, 0.1, n_splits=6)
    ws, used = tb.attn_decode_partial(cache, q, 1500, 0.1, n_splits=6)
    assert used == 6
    two = tb.attn_decode_merge(ws, 2, 16, used, sign_seed=4)
    assert torch.equal(one, two)
    # the partial states follow the documented layout: merging them on the
    # host reproduces the output
    wsf = ws[:2 * 16 * 6 * 130 * 4].view(torch.float32).view(2, 16, 6, 130).cpu().double().numpy()
    M = wsf[..., 0].max(axis=2, keepdims=True)
    wgt = np.exp2(wsf[..., 0:1] - M[..., None])
    L = (wgt[..., 0] * wsf[..., 1]).sum(axis=2)
    Or = (wgt * wsf[..., 2:]).sum(axis=2) / L[..., None]
    host = o.unrotate(Or, o.sign_vector(4))
    np.testing.assert_allclose(host, one.float().cpu().numpy(), atol=2e-3)


def test_timed_partial_matches_and_records_events():
    """The timed variant writes the same partial states and its dispatch
    records both events (elapsed time positive and finite)."""
    import ctypes
    rt = ctypes.CDLL("libamdhip64.so.7")
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                       ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
    rng = np.random.default_rng(22)
    k = rng.standard_normal((1, 2000, 2, 128)).astype(np.float32)
    cache = tb.KVCache(1, 2, 2000)
    _fill(cache, k, k)
    q = torch.from_numpy(rng.standard_normal((1, 16, 128)).astype(np.float32)).cuda()
    ws0, used0 = tb.attn_decode_partial(cache, q, 2000, 0.1, n_splits=5)
    ws1, used1 = tb.attn_decode_partial(cache, q, 2000, 0.1, n_splits=5,
                                        events=(ev[0].value, ev[1].value))
    torch.cuda.synchronize()
    n = 1 * 16 * 5 * 130 * 4
    assert used0 == used1 == 5
    assert torch.equal(ws0[:n], ws1[:n])
    ms = ctypes.c_float()
    assert rt.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 1000.0
    for e in ev:
        rt.hipEventDestroy(e)


@pytest.mark.parametrize("n_ctx", [33, 1000, 1023])
def test_unused_slots_with_nan_scales_do_not_leak(n_ctx):
    """Slots >= n_ctx of the last tile may hold anything; 0xFF bytes are NaN
    fp16 scales, which must not reach the output through p = 0."""
    rng = np.random.default_rng(40 + n_ctx)
    k = rng.standard_normal((1, n_ctx, 2, 128)).astype(np.float32)
    v = rng.standard_normal((1, n_ctx, 2, 128)).astype(np.float32)
    cache = tb.KVCache(1, 2, 1056)
    cache.k.fill_(0xFF)
    cache.v.fill_(0xFF)
    _fill(cache, k, v)
    kc, vc = _oracle_cache(k, v)
    q = rng.standard_normal((1, 16, 128)).astype(np.float32)
    ref = o.attn_decode_ref(q, kc, vc, n_ctx, 0.1)
    for P in (1, 3):
        out = tb.attn_decode(cache, torch.from_numpy(q).cuda(), n_ctx, 0.1, n_splits=P,
                             out_dtype=torch.float32)
        check_attn(out.cpu().numpy(), ref, False, f"nan tail n_ctx={n_ctx} P={P}")


@pytest.mark.parametrize("vmag", [1.0, 300.0, 5000.0])
@pytest.mark.parametrize("P", [2, 16])
def test_rising_scores_and_large_v_scales(vmag, P):
    """Scores that keep rising make the running maximum move through the
    whole context, so the reference maximum trails the scores by up to its
    lag; V blocks with scales above 256 (vmag 300, 5000) are where the lag
    must fall back to exact maxima, or P~ = p d^V would leave the fp16 range.
    Outputs are compared after dividing by vmag: the bar relative to the V
    values being averaged."""
    rng = np.random.default_rng(int(vmag) + P)
    B, H, G, T = 1, 2, 8, 4096
    q, k, v = rising_scores_inputs(rng, B, T, H, G, 1, vmag)
    cache = tb.KVCache(B, H, T, sign_seed=3)
    _fill(cache, k, v)
    kc, vc = _oracle_cache(k, v, 3)
    out = tb.attn_decode(cache, torch.from_numpy(q[:, 0]).cuda(), T, 1 / math.sqrt(128),
                         n_splits=P, out_dtype=torch.float32).cpu().numpy()
    ref = o.attn_decode_ref(q[:, 0], kc, vc, T, 1 / math.sqrt(128), 3)
    check_attn(out / vmag, ref / vmag, False, f"vmag={vmag} P={P}")
    if vmag <= 300.0:   # and at the bare absolute bound while |V| stays in the hundreds
        check_attn(out, ref, False, f"bare bound vmag={vmag} P={P}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_bf16_queries(out_dtype):
    """bf16 queries (16-bit patterns widened exactly to fp32 in the kernel);
    the oracle takes the same bf16 values."""
    out, ref = _run_small(2, 2, 8, 1000, 1000, 1000, 1 / math.sqrt(128), seed=6, P=0,
                          q_dtype=torch.bfloat16, out_dtype=out_dtype, rng_seed=8)
    check_attn(out, ref, out_dtype == torch.float16, "bf16 q")
