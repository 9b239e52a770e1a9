"""The no-allocation decode entry point against tbq4_attn_decode (GPU).

tbq4_attn_decode_noalloc is for callers that cannot allocate device memory:
its split-K partial states live in the library's static per-device scratch
array instead of a caller workspace.  Called here through the C ABI (ctypes
on libtbq4.so) with preallocated outputs, twice in a row -- the second call
smaller -- and compared with tbq4_attn_decode on the same inputs (the same
kernels and split count: identical outputs) and with the fp64 oracle (max-abs
2e-3, relative L2 1e-3, plus half an fp16 ulp for fp16 output).
"""

import ctypes

import numpy as np
import pytest
import torch

import long_context_attention_tbq4_amd as tb
from long_context_attention_tbq4_amd import _lib
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu

_DT = {torch.float32: _lib.F32, torch.float16: _lib.F16, torch.bfloat16: _lib.BF16}


def _noalloc(cache, q, n_ctx, scale, out, n_splits):
    d = cache.descriptor()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return _lib.lib().tbq4_attn_decode_noalloc(
        ctypes.byref(d), ctypes.c_void_p(q.data_ptr()), _DT[q.dtype], q.shape[1], n_ctx,
        float(scale), ctypes.c_void_p(out.data_ptr()), _DT[out.dtype], n_splits, stream)


def _case(seed, B, H, G, T, n_ctx, P, q_dtype, out_dtype):
    rng = np.random.default_rng([11, seed])
    k = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    v = rng.standard_normal((B, T, H, 128)).astype(np.float32)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    cache = tb.KVCache(B, H, ((T + 7) // 8) * 8, sign_seed=seed)
    tb.quantize_append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0)
    qt = torch.from_numpy(q).to(q_dtype).cuda()
    out = torch.full((B, H * G, 128), float("nan"), dtype=out_dtype, device="cuda")
    assert _noalloc(cache, qt, n_ctx, 0.1, out, P) == _lib.OK
    want = tb.attn_decode(cache, qt, n_ctx, 0.1, n_splits=P, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    kc = o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0]
    vc = o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0]
    ref = o.attn_decode_ref(qt.float().cpu().numpy(), kc, vc, n_ctx, 0.1, seed)
    check_attn(out.float().cpu().numpy(), ref, out_dtype == torch.float16, f"noalloc seed={seed}")


def test_noalloc_matches_decode_twice_second_smaller():
    # first call: 4 sequences x 8 KV heads, automatic split count
    _case(1, 4, 8, 8, 5000, 5000, 0, torch.float32, torch.float16)
    # second call, smaller: the array keeps the first call's contents
    _case(2, 1, 2, 4, 700, 650, 3, torch.float16, torch.float32)


def test_noalloc_rejects_partials_beyond_the_array():
    B, H, G, T = 4, 8, 8, 40000
    cache = tb.KVCache(B, H, T)
    q = torch.zeros((B, H * G, 128), dtype=torch.float32, device="cuda")
    out = torch.full((B, H * G, 128), 7.0, dtype=torch.float16, device="cuda")
    # 4 * 64 * 1024 * 520 bytes > 16 MiB
    assert _noalloc(cache, q, T, 0.1, out, 1024) == _lib.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # the largest split count that fits runs
    P = (_lib.NOALLOC_SCRATCH_BYTES // (B * H * G * 520))
    assert _noalloc(cache, q, T, 0.1, out, P) == _lib.OK
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
