"""GPU quantise-append parity: packed bytes must be identical to the oracle's.

Block format: page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Od czego zacząłem".
"""

import json
import os

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _special_blocks():
    rng = np.random.default_rng(100)
    x = [np.zeros(128), np.full(128, 1e30), np.full(128, -3e-30), np.full(128, 65504.0),
         np.full(128, 70000.0), np.full(128, 1e-8)]
    for j in (0, 1, 2, 63, 64, 127):
        e = np.zeros(128)
        e[j] = 1.0
        x.append(e)
        x.append(-7.0 * e)
    x.append(rng.standard_normal(128) * 1e-4)
    x.append(np.concatenate([np.ones(64), -np.ones(64)]))
    return np.array(x)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_quantize_blocks_bitexact_random(dtype):
    rng = np.random.default_rng(101)
    n = 20000
    x = np.concatenate([
        rng.standard_normal((n // 2, 128)),
        rng.standard_t(3, size=(n // 4, 128)) * rng.uniform(0.01, 100, size=(n // 4, 1)),
        rng.standard_normal((n // 4, 128)) * 10.0 ** rng.uniform(-6, 4, size=(n // 4, 1)),
    ])
    xt = torch.from_numpy(np.clip(x, -6e4, 6e4)).to(dtype)
    exact = xt.float().numpy()           # the values the library actually sees
    for seed in (0, 7):
        got = tb.quantize_blocks(xt.cuda(), sign_seed=seed).cpu().numpy()
        want = o.quantize_blocks(exact, seed=seed)[0]
        bad = np.nonzero(np.any(got != want, axis=1))[0]
        assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"


def test_quantize_special_blocks():
    x = _special_blocks().astype(np.float32)
    got = tb.quantize_blocks(torch.from_numpy(x).cuda()).cpu().numpy()
    want = o.quantize_blocks(x)[0]
    assert np.array_equal(got, want)


def test_golden_blocks():
    with open(os.path.join(GOLD, "known_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        x = np.zeros(128, np.float32)
        if blk["input"]["kind"] == "unit":
            x[blk["input"]["index"]] = blk["input"]["value"]
        got = tb.quantize_blocks(torch.from_numpy(x[None]).cuda(), sign_seed=blk["seed"])
        assert got.cpu().numpy()[0].tobytes().hex() == blk["hex"], blk["name"]


def test_append_layout_and_untouched_slots():
    B, H, cap = 2, 3, 48
    rng = np.random.default_rng(102)
    cache = tb.KVCache(B, H, cap, sign_seed=5)
    cache.k.fill_(0xAB)
    cache.v.fill_(0xCD)
    k1 = rng.standard_normal((B, 10, H, 128)).astype(np.float32)
    v1 = rng.standard_normal((B, 10, H, 128)).astype(np.float32)
    tb.quantize_append(cache, torch.from_numpy(k1).cuda(), torch.from_numpy(v1).cuda(), pos=17)
    k2 = rng.standard_normal((B, 3, H, 128)).astype(np.float32)
    tb.quantize_append(cache, torch.from_numpy(k2).cuda(), torch.from_numpy(k2).cuda(), pos=45)
    kc, vc = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    wk1 = o.quantize_blocks(k1.transpose(0, 2, 1, 3), seed=5)[0]
    wv1 = o.quantize_blocks(v1.transpose(0, 2, 1, 3), seed=5)[0]
    wk2 = o.quantize_blocks(k2.transpose(0, 2, 1, 3), seed=5)[0]
    assert np.array_equal(kc[:, :, 17:27], wk1)
    assert np.array_equal(vc[:, :, 17:27], wv1)
    assert np.array_equal(kc[:, :, 45:48], wk2)
    assert np.array_equal(vc[:, :, 45:48], wk2)
    untouched = np.ones(cap, bool)
    untouched[17:27] = False
    untouched[45:48] = False
    assert np.all(kc[:, :, untouched] == 0xAB) and np.all(vc[:, :, untouched] == 0xCD)


def test_append_capacity_overflow_is_an_error_and_writes_nothing():
    cache = tb.KVCache(1, 2, 16)
    x = torch.ones((1, 5, 2, 128), device="cuda")
    with pytest.raises(tb.TBQ4Error) as e:
        tb.quantize_append(cache, x, x, pos=12)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert int(cache.k.count_nonzero()) == 0 and int(cache.v.count_nonzero()) == 0


def test_append_is_deterministic():
    rng = np.random.default_rng(103)
    x = torch.from_numpy(rng.standard_normal((2, 64, 4, 128)).astype(np.float32)).cuda()
    a, b = tb.KVCache(2, 4, 64), tb.KVCache(2, 4, 64)
    tb.quantize_append(a, x, x, 0)
    tb.quantize_append(b, x, x, 0)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
