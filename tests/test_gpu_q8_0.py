"""GPU q8_0 cache rows against the oracle: stored bytes, then attention.

The pages name q8_0 as a KV cache type (the tgstat.ru channel @tech_di page's
server configuration sets K and V to q8_0) without defining it; the library
and the oracle read it as four 34-byte blocks per head vector (binary16 scale
d = amax/127, 32 int8 codes round(x/d) with halves away from zero, decided in
fp32).  Page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Konfiguracja": K and V types are chosen
separately, so TBQ4 K with q8_0 V and the reverse are run at the 128K decode
shape.  Bar: bytes bit-exact; outputs within max-abs 2e-3 (+ half an fp16 ulp
for fp16 output) and relative L2 1e-3.
"""

import json
import os

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from workloads import WORKLOADS, kv_rows, kv_tensor, q_decode
from _util import check_attn

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_q8(x):
    """Rows x [n][128] (torch, any accepted dtype) -> q8_0 rows [n][136]
    written by the append kernel (one sequence, one KV head)."""
    n = x.shape[0]
    cap = ((n + 7) // 8) * 8
    cache = tb.MixedKVCache(1, 1, cap, tb.FMT_Q8_0, tb.FMT_Q8_0)
    xs = x.reshape(1, n, 1, 128).contiguous().cuda()
    tb.mixed_append(cache, xs, xs, 0)
    torch.cuda.synchronize()
    k, v = cache.k[0, 0, :n].cpu().numpy(), cache.v[0, 0, :n].cpu().numpy()
    assert np.array_equal(k, v)
    assert not cache.k[0, 0, n:].any()
    return k


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_q8_rows_bitexact_random(dtype):
    rng = np.random.default_rng(401)
    n = 12000
    x = np.concatenate([
        rng.standard_normal((n // 2, 128)),
        rng.standard_t(3, size=(n // 4, 128)) * rng.uniform(0.01, 100, size=(n // 4, 1)),
        rng.standard_normal((n // 4, 128)) * 10.0 ** rng.uniform(-6, 4, size=(n // 4, 1)),
    ])
    xt = torch.from_numpy(np.clip(x, -6e4, 6e4)).to(dtype)
    exact = xt.float().numpy()           # the values the library actually sees
    got = _gpu_q8(xt)
    want = o.q8_0_rows(exact)
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"


def test_q8_special_rows_and_ties():
    rows = [np.zeros(128), np.full(128, 1e30), np.full(128, -3e-30), np.full(128, 65504.0),
            np.full(128, 1e-8)]
    t = np.zeros(128)
    t[:8] = [127, 0.5, -0.5, 1.5, -1.5, 2.5, 126.5, -126.5]    # d = 1: every half is a tie
    rows.append(t)
    t = np.zeros(128)
    t[32:40] = [254, 1, 3, -3, 5, -5, 7, 9]                      # d = 2
    rows.append(t)
    rng = np.random.default_rng(402)
    ties = np.round(rng.uniform(-126, 126, size=(1, 128)) * 2) / 2   # many exact halves
    ties[0, ::32] = 127.0
    rows.append(ties[0])
    x = np.array(rows, np.float32)
    assert np.array_equal(_gpu_q8(torch.from_numpy(x)), o.q8_0_rows(x))


def test_q8_golden_blocks():
    with open(os.path.join(GOLD, "known_rows_q8_0.json")) as f:
        blocks = json.load(f)["rows"]
    for blk in blocks:
        x = np.zeros(128, np.float32)
        k = blk["block"]
        x[32 * k:32 * k + len(blk["values"])] = blk["values"]
        got = _gpu_q8(torch.from_numpy(x[None]))[0]
        assert got[34 * k:34 * (k + 1)].tobytes().hex() == blk["hex"], blk["name"]


@pytest.mark.slow
@pytest.mark.parametrize("kf,vf", [(tb.FMT_TBQ4, tb.FMT_Q8_0), (tb.FMT_Q8_0, tb.FMT_TBQ4)])
def test_decode128k_tbq4_with_q8_sampled(kf, vf):
    """The 128K decode shape (batch 4, 8 / 64 heads) with one tensor TBQ4 and
    the other q8_0: two (sequence, KV head) rows re-quantised by the oracle,
    bytes and outputs checked."""
    w = WORKLOADS["decode128k"]
    T = w.n_ctx
    cache = tb.MixedKVCache(w.batch, w.n_kv_heads, T, kf, vf)
    for t0 in range(0, T, 32768):
        k = kv_tensor(w, 0, 0, t0, t0 + 32768)
        v = kv_tensor(w, 0, 1, t0, t0 + 32768)
        tb.mixed_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), t0)
    q = q_decode(w, 0, 0)
    out = tb.mixed_attn_decode(cache, torch.from_numpy(q).cuda(), T, w.softmax_scale).float().cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads

    def oracle(fmt, rows):
        if fmt == tb.FMT_TBQ4:
            b = o.quantize_blocks(rows)[0]
            return b, o.dequantize_blocks(b)
        b = o.q8_0_rows(rows)
        return b, o.dequantize_q8_0(b)

    for (b, g) in ((1, 6), (3, 0)):
        kc, kh = oracle(kf, kv_rows(w, 0, 0, b, g, 0, T))
        vc, vh = oracle(vf, kv_rows(w, 0, 1, b, g, 0, T))
        assert np.array_equal(cache.k[b, g].cpu().numpy(), kc), f"K bytes b={b} g={g}"
        assert np.array_equal(cache.v[b, g].cpu().numpy(), vc), f"V bytes b={b} g={g}"
        ref = o.attn_decode_rows_ref(q[b, g * G:(g + 1) * G], kh, vh, w.softmax_scale)
        check_attn(out[b, g * G:(g + 1) * G], ref, True, f"128k k{kf} v{vf} b={b} g={g}")
