"""Device-side lengths and graph-stable decode against the fp64 oracle.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "2. Mniej przechwyceń grafu CUDA": fewer graph re-captures as the
context grows.  Here the append positions and the attended lengths are read
from device memory, so one captured graph of (append, attend) replays while
the lengths advance.  Bar: appended blocks byte-identical to the oracle's,
outputs within max-abs 2e-3 (+ half an fp16 ulp) and relative L2 1e-3.
"""

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu


def _ref_rows(q, kc, vc, scale, seed=0):
    """q [G][128]; kc, vc [L][66] packed rows of one (sequence, KV head) of a
    cache with sign seed `seed`."""
    return o.attn_decode_rows_ref(q, o.dequantize_blocks(kc, seed), o.dequantize_blocks(vc, seed),
                                  scale)


def test_ragged_batch_append_at_and_varlen_decode():
    rng = np.random.default_rng(31)
    B, H, G, cap = 4, 2, 4, 2048
    lens = [2000, 37, 1025, 0]
    k = rng.standard_normal((B, cap, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, cap, H, 128)).astype(np.float32)
    cache = tb.KVCache(B, H, cap, sign_seed=5)
    # prefix [0, 1536) for every sequence through the host-position call
    tb.quantize_append(cache, torch.from_numpy(k[:, :1536].copy()).cuda(),
                       torch.from_numpy(v[:, :1536].copy()).cuda(), 0)
    # then 1-token appends at per-sequence positions: sequence 0 fills
    # 1536..1999, the others write one slot each or are skipped (position
    # at the capacity)
    before = cache.k.clone()
    fresh_k = rng.standard_normal((B, H, 128)).astype(np.float32)   # rows that differ from
    fresh_v = rng.standard_normal((B, H, 128)).astype(np.float32)   # what the slot held
    for t in range(1536, 2000):
        pos = [t, 36 if t == 1536 else cap, 1024 if t == 1536 else cap, cap]
        kn = np.stack([k[b, t] if b == 0 else fresh_k[b] for b in range(B)])[:, None]
        vn = np.stack([v[b, t] if b == 0 else fresh_v[b] for b in range(B)])[:, None]
        tb.quantize_append_at(cache, torch.from_numpy(np.ascontiguousarray(kn)).cuda(),
                              torch.from_numpy(np.ascontiguousarray(vn)).cuda(),
                              torch.tensor(pos, dtype=torch.int32, device="cuda"))
    k[1, 36], v[1, 36] = fresh_k[1], fresh_v[1]        # expected contents
    k[2, 1024], v[2, 1024] = fresh_k[2], fresh_v[2]
    torch.cuda.synchronize()
    kc_all = cache.k.cpu().numpy()
    vc_all = cache.v.cpu().numpy()
    # sequence 3 was never written past the prefix
    assert np.array_equal(kc_all[3, :, 1536:], before[3, :, 1536:].cpu().numpy())
    for b in range(3):
        n = lens[b]
        for g in range(H):
            kref = o.quantize_blocks(k[b, :n, g], 5)[0]
            vref = o.quantize_blocks(v[b, :n, g], 5)[0]
            assert np.array_equal(kc_all[b, g, :n], kref), (b, g)
            assert np.array_equal(vc_all[b, g, :n], vref), (b, g)

    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    qt = torch.from_numpy(q).cuda()
    scale = 0.1
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for P in (0, 1, 7, 64):
        out = tb.attn_decode_varlen(cache, qt, lens_t, cap, scale, n_splits=P,
                                    out_dtype=torch.float32).cpu().numpy()
        for b in range(B):
            n = lens[b]
            for g in range(H):
                got = out[b, g * G:(g + 1) * G]
                if n == 0:
                    assert np.array_equal(got, np.zeros_like(got)), "zero-length sequence"
                    continue
                ref = _ref_rows(q[b, g * G:(g + 1) * G], kc_all[b, g, :n], vc_all[b, g, :n], scale,
                                seed=5)
                check_attn(got, ref, False, f"varlen b={b} g={g} P={P}")

    # lengths above max_ctx are clamped to it
    lens_big = torch.tensor([2048, 2048, 2048, 2048], dtype=torch.int32, device="cuda")
    out = tb.attn_decode_varlen(cache, qt, lens_big, 1100, scale, n_splits=5,
                                out_dtype=torch.float32).cpu().numpy()
    for g in range(H):
        ref = _ref_rows(q[2, g * G:(g + 1) * G], kc_all[2, g, :1100], vc_all[2, g, :1100], scale,
                        seed=5)
        check_attn(out[2, g * G:(g + 1) * G], ref, False, "clamped to max_ctx")


def test_varlen_equals_fixed_length_call():
    """With every length equal to n_ctx the varlen call is the plain call."""
    rng = np.random.default_rng(32)
    B, H, T = 2, 2, 1000
    k = torch.from_numpy(rng.standard_normal((B, T, H, 128)).astype(np.float32)).cuda()
    cache = tb.KVCache(B, H, 1024)
    tb.quantize_append(cache, k, k, 0)
    q = torch.from_numpy(rng.standard_normal((B, 16, 128)).astype(np.float32)).cuda()
    a = tb.attn_decode(cache, q, T, 0.1, n_splits=9)
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    b = tb.attn_decode_varlen(cache, q, lens, T, 0.1, n_splits=9)
    assert torch.equal(a, b)


def test_graph_captured_decode_loop():
    """Capture (append at device positions, attend device lengths, advance)
    once; replay it step after step with new inputs; every replay matches
    the oracle and the appended blocks are the oracle's bytes."""
    rng = np.random.default_rng(33)
    B, H, G, cap, steps = 2, 2, 8, 4096, 6
    start = [1500, 700]
    hist_k = rng.standard_normal((B, cap, H, 128)).astype(np.float32)
    hist_v = rng.standard_normal((B, cap, H, 128)).astype(np.float32)
    cache = tb.KVCache(B, H, cap)
    tb.quantize_append(cache, torch.from_numpy(hist_k[:, :1500].copy()).cuda(),
                       torch.from_numpy(hist_v[:, :1500].copy()).cuda(), 0)
    pos = torch.tensor(start, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    k_new = torch.zeros((B, 1, H, 128), dtype=torch.float32, device="cuda")
    v_new = torch.zeros_like(k_new)
    q = torch.zeros((B, H * G, 128), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, H * G, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(tb.decode_workspace_bytes(B, H, H * G, cap, 32), dtype=torch.uint8,
                     device="cuda")
    scale = 1 / np.sqrt(128)

    def step():
        tb.quantize_append_at(cache, k_new, v_new, pos)
        torch.add(pos, 1, out=lens)
        tb.attn_decode_varlen(cache, q, lens, cap, scale, n_splits=32, out=out, workspace=ws)
        pos.add_(1)

    # warm up on a side stream (as graph capture requires), then capture;
    # the warm-up appends at 1500 / 700 and advances pos, so rewind it
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    pos.copy_(torch.tensor(start, dtype=torch.int32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    pos.copy_(torch.tensor(start, dtype=torch.int32))
    torch.cuda.synchronize()

    for i in range(steps):
        p = [start[b] + i for b in range(B)]
        for b in range(B):   # fresh rows (sequence 1's slots already held prefix rows)
            hist_k[b, p[b]] = rng.standard_normal((H, 128)).astype(np.float32)
            hist_v[b, p[b]] = rng.standard_normal((H, 128)).astype(np.float32)
            k_new[b, 0].copy_(torch.from_numpy(hist_k[b, p[b]]))
            v_new[b, 0].copy_(torch.from_numpy(hist_v[b, p[b]]))
        qh = rng.standard_normal((B, H * G, 128)).astype(np.float32)
        q.copy_(torch.from_numpy(qh))
        g.replay()
        torch.cuda.synchronize()                  # eager work between replays
        assert pos.cpu().tolist() == [p[b] + 1 for b in range(B)]
        got = out.cpu().numpy()
        kc_all = cache.k.cpu().numpy()
        vc_all = cache.v.cpu().numpy()
        for b in range(B):
            n = p[b] + 1
            for hk in range(H):
                # the new slot holds the oracle's block of this step's row
                assert np.array_equal(kc_all[b, hk, p[b]], o.quantize_blocks(hist_k[b, p[b], hk][None])[0][0])
                assert np.array_equal(vc_all[b, hk, p[b]], o.quantize_blocks(hist_v[b, p[b], hk][None])[0][0])
                ref = _ref_rows(qh[b, hk * G:(hk + 1) * G], kc_all[b, hk, :n], vc_all[b, hk, :n], scale)
                check_attn(got[b, hk * G:(hk + 1) * G], ref, False, f"replay {i} b={b} g={hk}")
