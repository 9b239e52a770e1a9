"""GPU TBQ3 cache against the oracle: stored bytes, then attention.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "6. Ten sam cache na Apple silicon": a TBQ3 KV cache runs beside TBQ4,
and its 3-bit packing needed a fix -- so the bytes the GPU writes are compared
with the oracle's one by one (bit-exact), for every input dtype, special
blocks and the hand-derived golden blocks, with every code at each of the 128
positions (32 of them straddle a byte boundary).  Attention on a TBQ3 cache:
max-abs 2e-3 (+ half an fp16 ulp for fp16 output) and relative L2 1e-3
against the fp64 definition on the dequantised tensors.
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


def _gpu_tbq3(x, seed=0):
    """Rows x [n][128] (torch, any accepted dtype) -> TBQ3 blocks [n][50]
    written by the append kernel (one sequence, one KV head)."""
    n = x.shape[0]
    cap = ((n + 7) // 8) * 8
    cache = tb.MixedKVCache(1, 1, cap, tb.FMT_TBQ3, tb.FMT_TBQ3, sign_seed=seed)
    xs = x.reshape(1, n, 1, 128).contiguous().cuda()
    tb.mixed_append(cache, xs, xs, 0)
    torch.cuda.synchronize()
    k, v = cache.k[0, 0, :n].cpu().numpy(), cache.v[0, 0, :n].cpu().numpy()
    assert np.array_equal(k, v)
    assert not cache.k[0, 0, n:].any()
    return k


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_tbq3_blocks_bitexact_random(dtype):
    rng = np.random.default_rng(301)
    n = 12000
    x = np.concatenate([
        rng.standard_normal((n // 2, 128)),
        rng.standard_t(3, size=(n // 4, 128)) * rng.uniform(0.01, 100, size=(n // 4, 1)),
        rng.standard_normal((n // 4, 128)) * 10.0 ** rng.uniform(-6, 4, size=(n // 4, 1)),
    ])
    xt = torch.from_numpy(np.clip(x, -6e4, 6e4)).to(dtype)
    exact = xt.float().numpy()           # the values the library actually sees
    for seed in (0, 7):
        got = _gpu_tbq3(xt, seed)
        want = o.quantize_blocks3(exact, seed=seed)[0]
        bad = np.nonzero(np.any(got != want, axis=1))[0]
        assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"
        # every code occurs at every one of the 128 positions (32 of which
        # straddle a byte boundary), so each 3-bit field is exercised
        codes = o.unpack3(want[:, 2:])
        assert all(np.unique(codes[:, i]).size == 8 for i in range(128))


def test_tbq3_special_blocks():
    rng = np.random.default_rng(302)
    x = [np.zeros(128), np.full(128, 1e30), np.full(128, -3e-30), np.full(128, 65504.0),
         np.full(128, 70000.0), np.full(128, 1e-8), rng.standard_normal(128) * 1e-4,
         np.concatenate([np.ones(64), -np.ones(64)])]
    for j in (0, 1, 2, 63, 64, 127):
        e = np.zeros(128)
        e[j] = 1.0
        x += [e, -7.0 * e]
    x = np.array(x, np.float32)
    assert np.array_equal(_gpu_tbq3(torch.from_numpy(x)), o.quantize_blocks3(x)[0])


def test_tbq3_golden_blocks():
    with open(os.path.join(GOLD, "known_blocks_tbq3.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        x = np.zeros(128, np.float32)
        if blk["input"]["kind"] == "unit":
            x[blk["input"]["index"]] = blk["input"]["scale"]
        got = _gpu_tbq3(torch.from_numpy(x[None]), blk["seed"])
        assert got[0].tobytes().hex() == blk["hex"], blk["name"]


@pytest.mark.slow
def test_decode128k_tbq3_sampled():
    """The 128K decode shape (batch 4, 8 / 64 heads) on a TBQ3 K and V cache:
    two (sequence, KV head) rows re-quantised by the oracle, bytes and
    outputs checked."""
    w = WORKLOADS["decode128k"]
    T = w.n_ctx
    cache = tb.MixedKVCache(w.batch, w.n_kv_heads, T, tb.FMT_TBQ3, tb.FMT_TBQ3)
    for t0 in range(0, T, 32768):
        k = kv_tensor(w, 0, 0, t0, t0 + 32768)
        v = kv_tensor(w, 0, 1, t0, t0 + 32768)
        tb.mixed_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), t0)
    q = q_decode(w, 0, 0)
    out = tb.mixed_attn_decode(cache, torch.from_numpy(q).cuda(), T, w.softmax_scale).float().cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    for (b, g) in ((0, 5), (2, 1)):
        kc = o.quantize_blocks3(kv_rows(w, 0, 0, b, g, 0, T))[0]
        vc = o.quantize_blocks3(kv_rows(w, 0, 1, b, g, 0, T))[0]
        assert np.array_equal(cache.k[b, g].cpu().numpy(), kc), f"K bytes b={b} g={g}"
        assert np.array_equal(cache.v[b, g].cpu().numpy(), vc), f"V bytes b={b} g={g}"
        ref = o.attn_decode_rows_ref(q[b, g * G:(g + 1) * G], o.dequantize_blocks3(kc),
                                     o.dequantize_blocks3(vc), w.softmax_scale)
        check_attn(out[b, g * G:(g + 1) * G], ref, True, f"128k tbq3 b={b} g={g}")
