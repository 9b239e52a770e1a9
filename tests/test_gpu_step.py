"""The fused decode step (append one token, attend over the cache holding it)
against the oracle and against the two separate calls it replaces.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "Od czego zacząłem": the new token's K and V are quantised into the
TBQ4 cache and flash attention reads the raw blocks.  Bar: the cache bytes
identical to tbq4_quantize_append's (and so to the oracle's), outputs within
max-abs 2e-3 (+ half an fp16 ulp for fp16 outputs) and relative L2 1e-3 of
the fp64 oracle over slots [0, pos].
"""

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _ref(q_rows, kc, vc, n, scale, seed):
    """oracle attention of q_rows [G][128] over the first n packed rows"""
    return o.attn_decode_rows_ref(q_rows, o.dequantize_blocks(kc[:n], seed),
                                  o.dequantize_blocks(vc[:n], seed), scale)


def _prefix_cache(rng, B, H, cap, n, seed):
    k = rng.standard_normal((B, n, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, n, H, 128)).astype(np.float32)
    cache = tb.KVCache(B, H, cap, sign_seed=seed)
    if n:
        tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    return cache


def _clone(cache):
    c = tb.KVCache(cache.batch, cache.n_kv_heads, cache.capacity, sign_seed=cache.sign_seed)
    c.k.copy_(cache.k)
    c.v.copy_(cache.v)
    return c


@pytest.mark.parametrize("src,qdt", [("f32", "f32"), ("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("H,G", [(2, 4), (1, 8)])
def test_step_equals_append_then_decode(src, qdt, H, G):
    rng = np.random.default_rng(41)
    B, cap, pos, seed = 2, 2048, 1000, 3
    cache = _prefix_cache(rng, B, H, cap, pos, seed)
    twin = _clone(cache)
    kn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda().to(DT[src])
    vn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda().to(DT[src])
    q = torch.from_numpy(rng.standard_normal((B, H * G, 128)).astype(np.float32)).cuda().to(DT[qdt])
    scale = 0.09
    print(f"[step] src {src} q {qdt} H {H} G {G}", flush=True)
    out = tb.decode_step(cache, kn, vn, q, pos, scale, out_dtype=torch.float32)
    tb.quantize_append(twin, kn, vn, pos)
    torch.cuda.synchronize()
    assert torch.equal(cache.k, twin.k) and torch.equal(cache.v, twin.v), "stored bytes differ"
    sep = tb.attn_decode(twin, q, pos + 1, scale, out_dtype=torch.float32)
    kc, vc = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    qf = q.float().cpu().numpy()
    out, sep = out.cpu().numpy(), sep.cpu().numpy()
    for b in range(B):
        for g in range(H):
            ref = _ref(qf[b, g * G:(g + 1) * G], kc[b, g], vc[b, g], pos + 1, scale, seed)
            check_attn(out[b, g * G:(g + 1) * G], ref, False, f"step b={b} g={g}")
            check_attn(sep[b, g * G:(g + 1) * G], ref, False, f"append+decode b={b} g={g}")
    # the new token's bytes are the oracle's
    knf, vnf = kn.float().cpu().numpy(), vn.float().cpu().numpy()
    for b in range(B):
        for g in range(H):
            assert np.array_equal(kc[b, g, pos], o.quantize_blocks(knf[b, 0, g][None], seed)[0][0])
            assert np.array_equal(vc[b, g, pos], o.quantize_blocks(vnf[b, 0, g][None], seed)[0][0])


@pytest.mark.parametrize("pos", [0, 1, 31, 32, 33, 1023])
@pytest.mark.parametrize("P", [0, 1, 5, 64, 300])
def test_step_positions_and_splits(pos, P):
    """slot 0 (the token alone), tile edges, the last slot; split counts
    from one to more splits than tiles; fp16 output."""
    rng = np.random.default_rng(42 + pos)
    B, H, G, cap, seed = 2, 2, 4, 1024, 0
    cache = _prefix_cache(rng, B, H, cap, pos, seed)
    kn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda()
    vn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda()
    q = torch.from_numpy(rng.standard_normal((B, H * G, 128)).astype(np.float32)).cuda()
    print(f"[step] pos {pos} P {P}", flush=True)
    out = tb.decode_step(cache, kn, vn, q, pos, 0.1, n_splits=P).float().cpu().numpy()
    kc, vc, qf = cache.k.cpu().numpy(), cache.v.cpu().numpy(), q.cpu().numpy()
    for b in range(B):
        for g in range(H):
            ref = _ref(qf[b, g * G:(g + 1) * G], kc[b, g], vc[b, g], pos + 1, 0.1, seed)
            check_attn(out[b, g * G:(g + 1) * G], ref, True, f"pos={pos} P={P} b={b} g={g}")


def test_step_dominant_new_token():
    """A new key aligned with the queries carries almost all the weight: its
    partial state (written by the new-token wavefront) sets the maximum."""
    rng = np.random.default_rng(43)
    B, H, G, cap, pos, seed = 1, 2, 8, 4096, 3000, 9
    cache = _prefix_cache(rng, B, H, cap, pos, seed)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    kn = np.zeros((B, 1, H, 128), np.float32)
    for g in range(H):
        kn[0, 0, g] = 6.0 * q[0, g * G:(g + 1) * G].sum(axis=0) / np.sqrt(G)
    vn = (5.0 * rng.standard_normal((B, 1, H, 128))).astype(np.float32)
    out = tb.decode_step(cache, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                         torch.from_numpy(q).cuda(), pos, 0.088, out_dtype=torch.float32)
    out = out.cpu().numpy()
    kc, vc = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    for g in range(H):
        ref = _ref(q[0, g * G:(g + 1) * G], kc[0, g], vc[0, g], pos + 1, 0.088, seed)
        check_attn(out[0, g * G:(g + 1) * G], ref, False, f"dominant g={g}")


def test_step_device_positions():
    """Per-sequence slots from device memory, bounded by pos: a slot outside
    [0, pos] writes nothing and gives a zero output."""
    rng = np.random.default_rng(44)
    B, H, G, cap, seed, bound = 5, 2, 4, 2048, 6, 1500
    n = 1600
    cache = _prefix_cache(rng, B, H, cap, n, seed)
    before_k, before_v = cache.k.clone(), cache.v.clone()
    slots = [1200, 0, 1500, -1, 1550]          # the last two: outside [0, bound]
    kn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda()
    vn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda()
    q = torch.from_numpy(rng.standard_normal((B, H * G, 128)).astype(np.float32)).cuda()
    pos_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    out = tb.decode_step(cache, kn, vn, q, bound, 0.1, positions=pos_t, n_splits=7,
                         out_dtype=torch.float32).cpu().numpy()
    kc, vc, qf = cache.k.cpu().numpy(), cache.v.cpu().numpy(), q.cpu().numpy()
    bk, bv = before_k.cpu().numpy(), before_v.cpu().numpy()
    knf, vnf = kn.cpu().numpy(), vn.cpu().numpy()
    for b, s in enumerate(slots):
        if 0 <= s <= bound:
            mask = np.ones(cap, bool)
            mask[s] = False
            assert np.array_equal(kc[b][:, mask], bk[b][:, mask]), f"b={b}: other slots changed"
            for g in range(H):
                assert np.array_equal(kc[b, g, s], o.quantize_blocks(knf[b, 0, g][None], seed)[0][0])
                assert np.array_equal(vc[b, g, s], o.quantize_blocks(vnf[b, 0, g][None], seed)[0][0])
                ref = _ref(qf[b, g * G:(g + 1) * G], kc[b, g], vc[b, g], s + 1, 0.1, seed)
                check_attn(out[b, g * G:(g + 1) * G], ref, False, f"slot {s} b={b} g={g}")
        else:
            assert np.array_equal(kc[b], bk[b]) and np.array_equal(vc[b], bv[b]), f"b={b} written"
            assert np.array_equal(out[b], np.zeros_like(out[b])), f"b={b}: output not zero"


def test_step_graph_replays():
    """One captured graph of (step at device positions, advance the
    positions) replays step after step; each replay matches the oracle, with
    eager work and synchronisation between replays."""
    rng = np.random.default_rng(45)
    B, H, G, cap, seed, steps = 2, 2, 8, 4096, 2, 5
    start = 2000
    hist_k = rng.standard_normal((B, start + steps, H, 128)).astype(np.float32)
    hist_v = rng.standard_normal((B, start + steps, H, 128)).astype(np.float32)
    cache = tb.KVCache(B, H, cap, sign_seed=seed)
    tb.quantize_append(cache, torch.from_numpy(hist_k[:, :start].copy()).cuda(),
                       torch.from_numpy(hist_v[:, :start].copy()).cuda(), 0)
    pos_t = torch.full((B,), start, dtype=torch.int32, device="cuda")
    kn = torch.empty((B, 1, H, 128), dtype=torch.float32, device="cuda")
    vn = torch.empty_like(kn)
    q = torch.empty((B, H * G, 128), dtype=torch.float32, device="cuda")
    out = torch.empty((B, H * G, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(tb.decode_step_workspace_bytes(B, H, H * G, cap, 0), dtype=torch.uint8,
                     device="cuda")

    def body():
        tb.decode_step(cache, kn, vn, q, cap - 1, 0.1, positions=pos_t, out=out, workspace=ws)
        pos_t.add_(1)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # warm-up outside capture (writes slot `start`, redone below)
        kn.copy_(torch.from_numpy(hist_k[:, start:start + 1].copy()))
        vn.copy_(torch.from_numpy(hist_v[:, start:start + 1].copy()))
        q.normal_()
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    pos_t.fill_(start)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    for t in range(steps):
        p = start + t
        kn.copy_(torch.from_numpy(hist_k[:, p:p + 1].copy()))
        vn.copy_(torch.from_numpy(hist_v[:, p:p + 1].copy()))
        qn = rng.standard_normal((B, H * G, 128)).astype(np.float32)
        q.copy_(torch.from_numpy(qn))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert pos_t.cpu().tolist() == [p + 1] * B
        got = out.cpu().numpy()
        kc, vc = cache.k.cpu().numpy(), cache.v.cpu().numpy()
        for b in range(B):
            for h in range(H):
                assert np.array_equal(kc[b, h, p], o.quantize_blocks(hist_k[b, p, h][None], seed)[0][0])
                ref = _ref(qn[b, h * G:(h + 1) * G], kc[b, h], vc[b, h], p + 1, 0.1, seed)
                check_attn(got[b, h * G:(h + 1) * G], ref, False, f"replay {t} b={b} h={h}")


def test_step_timed_matches_and_records_events():
    """tbq4_decode_step_timed: the same output as the untimed call, and the
    two events its split-kernel dispatch records span a positive time."""
    import ctypes
    rt = ctypes.CDLL("libamdhip64.so.7")
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                       ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
    rng = np.random.default_rng(46)
    B, H, G, cap, pos = 2, 2, 4, 4096, 3000
    cache = _prefix_cache(rng, B, H, cap, pos, 1)
    kn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda()
    vn = torch.from_numpy(rng.standard_normal((B, 1, H, 128)).astype(np.float32)).cuda()
    q = torch.from_numpy(rng.standard_normal((B, H * G, 128)).astype(np.float32)).cuda()
    a = tb.decode_step(cache, kn, vn, q, pos, 0.1, out_dtype=torch.float32)
    b = tb.decode_step(cache, kn, vn, q, pos, 0.1, out_dtype=torch.float32,
                       events=(ev[0].value, ev[1].value))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ms = ctypes.c_float()
    assert rt.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 1000.0
    for e in ev:
        rt.hipEventDestroy(e)
