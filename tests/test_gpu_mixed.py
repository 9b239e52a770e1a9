"""Mixed K/V cache formats (TBQ4, TBQ3, q8_0 or fp16 per tensor) against the fp64 oracle.

Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
section "Konfiguracja": the K and the V cache types are chosen separately;
section "6. Ten sam cache na Apple silicon" adds a TBQ3 cache; the tgstat.ru
channel @tech_di page runs a q8_0 cache.  Each tensor is stored as TBQ4 or
TBQ3 blocks (rotated), q8_0 rows or binary16 rows (not rotated); attention is
the plain definition on the dequantised tensors.  Bar: stored bytes identical
to the oracle's; outputs within max-abs 2e-3 (+ half an fp16 ulp for fp16
output) and relative L2 1e-3.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu

ALL = list(itertools.product([tb.FMT_TBQ4, tb.FMT_F16, tb.FMT_TBQ3, tb.FMT_Q8_0], repeat=2))
MIXED = [f for f in ALL if f != (tb.FMT_TBQ4, tb.FMT_TBQ4)]


def _oracle_tensor(x, fmt, seed):
    """x: fp32 [B][T][H][128] -> (stored bytes [B][H][T][row], dequantised
    fp64 [B][H][T][128]) in the oracle's format."""
    xh = np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    if fmt == tb.FMT_TBQ4:
        packed = o.quantize_blocks(xh, seed)[0]
        return packed, o.dequantize_blocks(packed, seed)
    if fmt == tb.FMT_TBQ3:
        packed = o.quantize_blocks3(xh, seed)[0]
        return packed, o.dequantize_blocks3(packed, seed)
    if fmt == tb.FMT_Q8_0:
        rows = o.q8_0_rows(xh)
        return rows, o.dequantize_q8_0(rows)
    rows = o.f16_rows(xh)
    return rows.view(np.uint8), o.dequantize_f16(rows)


def _case(kf, vf, B, H, G, T, cap, scale, P, seed=0, rng_seed=0, kscale=1.0, junk=False,
          out_dtype=torch.float32):
    rng = np.random.default_rng(rng_seed)
    k = (rng.standard_normal((B, T, H, 128)) * kscale).astype(np.float32)
    v = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    cache = tb.MixedKVCache(B, H, cap, kf, vf, sign_seed=seed)
    if junk:   # unused slots: 0xFF bytes (NaN fp16 values / NaN TBQ4 scales)
        cache.k.fill_(0xFF)
        cache.v.fill_(0xFF)
    half = T // 2
    tb.mixed_append(cache, torch.from_numpy(k[:, :half].copy()).cuda(),
                    torch.from_numpy(v[:, :half].copy()).cuda(), 0)
    tb.mixed_append(cache, torch.from_numpy(k[:, half:].copy()).cuda(),
                    torch.from_numpy(v[:, half:].copy()).cuda(), half)
    kb, kh = _oracle_tensor(k, kf, seed)
    vb, vh = _oracle_tensor(v, vf, seed)
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kb), "K bytes"
    assert np.array_equal(cache.v[:, :, :T].cpu().numpy(), vb), "V bytes"
    out = tb.mixed_attn_decode(cache, torch.from_numpy(q).cuda(), T, scale, n_splits=P,
                               out_dtype=out_dtype).float().cpu().numpy()
    ref = np.empty_like(out, dtype=np.float64)
    for b in range(B):
        for g in range(H):
            ref[b, g * G:(g + 1) * G] = o.attn_decode_rows_ref(q[b, g * G:(g + 1) * G], kh[b, g],
                                                               vh[b, g], scale)
    return out, ref


@pytest.mark.parametrize("kf,vf", ALL)
@pytest.mark.parametrize("P", [0, 3])
def test_formats(kf, vf, P):
    out, ref = _case(kf, vf, 2, 2, 8, 700, 712, 1 / math.sqrt(128), P, seed=3, rng_seed=kf + 4 * vf)
    check_attn(out, ref, False, f"k{kf} v{vf} P={P}")


@pytest.mark.parametrize("kf,vf", MIXED)
def test_group_sizes_fp16_output_and_seed(kf, vf):
    for G in (1, 4):
        out, ref = _case(kf, vf, 1, 3, G, 1000, 1008, 0.1, 5, seed=11, rng_seed=G,
                         out_dtype=torch.float16)
        check_attn(out, ref, True, f"k{kf} v{vf} G={G}")


@pytest.mark.parametrize("kf,vf", MIXED)
def test_peaky_scores(kf, vf):
    out, ref = _case(kf, vf, 1, 1, 8, 2048, 2048, 1 / math.sqrt(128), 8, kscale=30.0, rng_seed=5)
    check_attn(out, ref, False, f"peaky k{kf} v{vf}")


@pytest.mark.parametrize("kf,vf", MIXED)
@pytest.mark.parametrize("T", [33, 1023])
def test_unused_slots_with_nan_do_not_leak(kf, vf, T):
    out, ref = _case(kf, vf, 1, 2, 8, T, 1056, 0.1, 2, rng_seed=T, junk=True)
    check_attn(out, ref, False, f"nan tail k{kf} v{vf} T={T}")


def test_tbq4_formats_match_the_tbq4_cache():
    """Both tensors TBQ4 through the mixed calls = the TBQ4-only calls."""
    rng = np.random.default_rng(9)
    k = torch.from_numpy(rng.standard_normal((2, 500, 2, 128)).astype(np.float32)).cuda()
    q = torch.from_numpy(rng.standard_normal((2, 16, 128)).astype(np.float32)).cuda()
    a = tb.KVCache(2, 2, 504, sign_seed=2)
    tb.quantize_append(a, k, k, 0)
    m = tb.MixedKVCache(2, 2, 504, tb.FMT_TBQ4, tb.FMT_TBQ4, sign_seed=2)
    tb.mixed_append(m, k, k, 0)
    assert torch.equal(a.k, m.k) and torch.equal(a.v, m.v)
    assert torch.equal(tb.attn_decode(a, q, 500, 0.1, n_splits=4),
                       tb.mixed_attn_decode(m, q, 500, 0.1, n_splits=4))


@pytest.mark.parametrize("kf,vf", ALL)
@pytest.mark.parametrize("B,H,n_new", [(1, 1, 1), (1, 3, 1), (1, 2, 17)])
def test_append_block_counts_not_multiple_of_four(kf, vf, B, H, n_new):
    """Appends whose block count is not a multiple of the 4 wavefronts of a
    quantiser workgroup: the extra wavefronts have no block and must not
    touch memory; the written slots hold the oracle's bytes."""
    rng = np.random.default_rng(50 + n_new)
    k = rng.standard_normal((B, n_new, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, n_new, H, 128)).astype(np.float32)
    cache = tb.MixedKVCache(B, H, 64, kf, vf, sign_seed=1)
    tb.mixed_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 5)
    torch.cuda.synchronize()
    kb, _ = _oracle_tensor(k, kf, 1)
    vb, _ = _oracle_tensor(v, vf, 1)
    assert np.array_equal(cache.k[:, :, 5:5 + n_new].cpu().numpy(), kb)
    assert np.array_equal(cache.v[:, :, 5:5 + n_new].cpu().numpy(), vb)
    assert not cache.k[:, :, :5].any() and not cache.k[:, :, 5 + n_new:].any()


@pytest.mark.parametrize("scale", [0.09, 1e-4, 2.0])
@pytest.mark.parametrize("kf,vf", ALL)
def test_prefill_formats(kf, vf, scale):
    """Prefill chunk (query i at n_past + i sees slots 0 .. n_past + i) on K
    and V stored as TBQ4, TBQ3, q8_0 or fp16, against the fp64 definition on
    the dequantised tensors; unused slots hold 0xFF bytes (NaN fp16 values,
    NaN scales) that must not leak.  The softmax scale sets the power of two
    that normalises q': at its bound for 0.09 and (far past it) 1e-4, inside
    its range for 2.0; TBQ K values carry it, fp16 and q8_0 K take it as
    their key scale."""
    rng = np.random.default_rng(40 + kf + 4 * vf)
    B, H, G, n_past, n_q, cap, seed = 2, 2, 4, 301, 97, 424, 5
    T = n_past + n_q
    k = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    q = rng.standard_normal((B, n_q, H * G, 128)).astype(np.float32)
    cache = tb.MixedKVCache(B, H, cap, kf, vf, sign_seed=seed)
    cache.k.fill_(0xFF)
    cache.v.fill_(0xFF)
    tb.mixed_append(cache, torch.from_numpy(k[:, :n_past].copy()).cuda(),
                    torch.from_numpy(v[:, :n_past].copy()).cuda(), 0)
    tb.mixed_append(cache, torch.from_numpy(k[:, n_past:].copy()).cuda(),
                    torch.from_numpy(v[:, n_past:].copy()).cuda(), n_past)
    kb, kh = _oracle_tensor(k, kf, seed)
    vb, vh = _oracle_tensor(v, vf, seed)
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kb), "K bytes"
    assert np.array_equal(cache.v[:, :, :T].cpu().numpy(), vb), "V bytes"
    out = tb.mixed_attn_prefill_chunk(cache, torch.from_numpy(q).cuda(), n_past, scale,
                                      out_dtype=torch.float32).cpu().numpy()
    ref = np.empty(out.shape, np.float64)
    for b in range(B):
        for g in range(H):
            for i in range(n_q):
                n = n_past + i + 1
                ref[b, i, g * G:(g + 1) * G] = o.attn_decode_rows_ref(
                    q[b, i, g * G:(g + 1) * G], kh[b, g, :n], vh[b, g, :n], scale)
    check_attn(out, ref, False, f"prefill k{kf} v{vf} scale {scale}")
    if (kf, vf) == (tb.FMT_TBQ4, tb.FMT_TBQ4):   # the TBQ4 call computes the same
        plain = tb.KVCache(B, H, cap, sign_seed=seed)
        plain.k.copy_(cache.k)
        plain.v.copy_(cache.v)
        same = tb.attn_prefill_chunk(plain, torch.from_numpy(q).cuda(), n_past, scale,
                                     out_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(same, out)


VERIFY_SHAPES = [   # B, H, G, n_past, n_q, cap, P
    (2, 2, 4, 301, 3, 320, 0),
    (1, 1, 8, 5, 4, 16, 1),
    (3, 2, 1, 70, 1, 80, 3),
    (1, 2, 8, 1000, 2, 1008, 4),
]


@pytest.mark.parametrize("kf,vf", ALL)
@pytest.mark.parametrize("shape", range(len(VERIFY_SHAPES)))
def test_verify_formats(kf, vf, shape):
    """Multi-query verify (query i at n_past + i sees slots 0 .. n_past + i)
    on K and V stored as TBQ4, TBQ3, q8_0 or fp16, against the fp64
    definition on the dequantised tensors; unused slots hold 0xFF bytes that
    must not leak."""
    B, H, G, n_past, n_q, cap, P = VERIFY_SHAPES[shape]
    rng = np.random.default_rng(70 + kf + 4 * vf + 16 * shape)
    seed, scale = 9 + shape, 0.1
    T = n_past + n_q
    k = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    q = rng.standard_normal((B, n_q, H * G, 128)).astype(np.float32)
    cache = tb.MixedKVCache(B, H, cap, kf, vf, sign_seed=seed)
    cache.k.fill_(0xFF)
    cache.v.fill_(0xFF)
    tb.mixed_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    kb, kh = _oracle_tensor(k, kf, seed)
    vb, vh = _oracle_tensor(v, vf, seed)
    assert np.array_equal(cache.k[:, :, :T].cpu().numpy(), kb), "K bytes"
    assert np.array_equal(cache.v[:, :, :T].cpu().numpy(), vb), "V bytes"
    out = tb.mixed_attn_verify(cache, torch.from_numpy(q).cuda(), n_past, scale, n_splits=P,
                               out_dtype=torch.float32).cpu().numpy()
    ref = np.empty(out.shape, np.float64)
    for b in range(B):
        for g in range(H):
            for i in range(n_q):
                n = n_past + i + 1
                ref[b, i, g * G:(g + 1) * G] = o.attn_decode_rows_ref(
                    q[b, i, g * G:(g + 1) * G], kh[b, g, :n], vh[b, g, :n], scale)
    check_attn(out, ref, False, f"verify k{kf} v{vf} shape {VERIFY_SHAPES[shape]}")
    if (kf, vf) == (tb.FMT_TBQ4, tb.FMT_TBQ4):   # the TBQ4 call computes the same
        plain = tb.KVCache(B, H, cap, sign_seed=seed)
        plain.k.copy_(cache.k)
        plain.v.copy_(cache.v)
        same = tb.attn_verify(plain, torch.from_numpy(q).cuda(), n_past, scale, n_splits=P,
                              out_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(same, out)
