"""Host-side checks of the C ABI (no GPU needed; no kernel is launched).

Every argument check of include/tbq4.h runs on the host before any launch,
so invalid calls can be exercised here; each must return its status code.
Capacity overflow must be an error, not a crash (page "Kontekst 262K na jednej
RTX 4090: co dodałem do llama.cpp-turboq", section "4. Poprawność w długich
sesjach": a full context is handled gracefully).
"""

import ctypes
import os
import re

import pytest

from long_context_attention_tbq4_amd import _lib
from oracle import tbq4_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_library_exports_every_declared_symbol(L):
    with open(os.path.join(ROOT, "include", "tbq4.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(tbq4_[a-z_0-9]+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_library_exports_the_measurement_helpers(L):
    with open(os.path.join(ROOT, "include", "tbq4_bench.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(tbq4_[a-z_0-9]+)\s*\(", header))
    assert declared == set(_lib.BENCH_EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    # argument checks run before any launch
    assert L.tbq4_bench_stream_read(None, 1 << 20, FAKE, 64, None) == -1
    assert L.tbq4_bench_stream_read(FAKE, 24, FAKE, 64, None) == -1
    assert L.tbq4_bench_stream_read(FAKE, 1 << 20, FAKE, 0, None) == -1
    assert L.tbq4_bench_mfma_f16(0, FAKE, 64, None) == -1
    assert L.tbq4_bench_mfma_f16(10, None, 64, None) == -1


def test_version_and_status_strings(L):
    assert L.tbq4_version().decode().count(".") == 2
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.tbq4_status_str(s)
    assert L.tbq4_status_str(-99) == b"unknown status"


def test_cache_bytes_reproduces_page_footprint(L):
    # 262144 tokens, 128 (layer, kv head) pairs, K and V: 4.125 GiB (printed
    # as about 4.1 GiB), against 16 GiB for an FP16 cache.
    per = L.tbq4_cache_bytes(1, 128, 262144)
    assert per == 262144 * 128 * 66
    assert 2 * per / 2 ** 30 == 4.125
    assert L.tbq4_cache_bytes(-1, 1, 8) == 0


def test_sign_vector_matches_oracle(L):
    for seed in (0, 1, 2, 12345, 2 ** 64 - 1):
        buf = (ctypes.c_uint8 * 16)()
        assert L.tbq4_sign_vector(seed, buf) == 0
        assert bytes(buf) == o.sign_bits(seed)
    assert L.tbq4_sign_vector(0, None) == _lib.ERR_INVALID_ARG


def test_workspace_and_splits(L):
    p = L.tbq4_decode_auto_splits(4, 8, 131072)
    assert 1 <= p <= 1024
    assert L.tbq4_decode_workspace_bytes(4, 8, 64, 131072, 0) >= 4 * 64 * p * 130 * 4
    assert L.tbq4_decode_workspace_bytes(4, 8, 64, 131072, 16) == 4 * 64 * 16 * 130 * 4
    assert L.tbq4_decode_workspace_bytes(4, 8, 64, 131072, 1025) == 0
    assert L.tbq4_decode_auto_splits(0, 8, 100) == 0


FAKE = 0x10000  # a 16-byte aligned, never dereferenced address


def _cache(batch=1, heads=2, head_dim=128, cap=64, k=FAKE, v=FAKE, seed=0):
    return _lib.Cache(k, v, batch, heads, head_dim, cap, seed)


def test_append_argument_errors(L):
    c = _cache()
    app = L.tbq4_quantize_append
    assert app(None, FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(_cache(head_dim=64)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_UNSUPPORTED
    assert app(ctypes.byref(_cache(cap=60)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_ALIGNMENT
    assert app(ctypes.byref(_cache(k=FAKE + 2)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_ALIGNMENT
    assert app(ctypes.byref(_cache(k=0)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(c), FAKE, FAKE, 7, 0, 1, None) == _lib.ERR_INVALID_ARG    # dtype
    assert app(ctypes.byref(c), FAKE, FAKE, 0, 60, 5, None) == _lib.ERR_CAPACITY      # 65 > 64
    assert app(ctypes.byref(c), FAKE, FAKE, 0, 64, 1, None) == _lib.ERR_CAPACITY
    assert app(ctypes.byref(c), FAKE, FAKE, 0, -1, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(c), None, FAKE, 0, 0, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(c), FAKE + 4, FAKE, 0, 0, 1, None) == _lib.ERR_ALIGNMENT
    # n_new = 0 is a valid no-op that launches nothing
    assert app(ctypes.byref(c), None, None, 0, 64, 0, None) == _lib.OK


def test_decode_argument_errors(L):
    c = _cache(heads=2, cap=64)
    ws = 1 << 20

    def dec(cache=c, q=FAKE, qdt=0, hq=8, n_ctx=10, scale=1.0, out=FAKE, odt=1, p=0,
            w=FAKE, wb=ws):
        return L.tbq4_attn_decode(ctypes.byref(cache) if cache is not None else None, q, qdt, hq,
                                  n_ctx, scale, out, odt, p, w, wb, None)
    assert dec(cache=None) == _lib.ERR_INVALID_ARG
    assert dec(q=None) == _lib.ERR_INVALID_ARG
    assert dec(qdt=3) == _lib.ERR_INVALID_ARG          # no such dtype
    assert dec(odt=2) == _lib.ERR_INVALID_ARG
    assert dec(hq=7) == _lib.ERR_UNSUPPORTED            # not a multiple of 2 kv heads
    assert dec(hq=18) == _lib.ERR_UNSUPPORTED           # group of 9 > 8
    assert dec(n_ctx=0) == _lib.ERR_CAPACITY
    assert dec(n_ctx=65) == _lib.ERR_CAPACITY
    assert dec(p=1025) == _lib.ERR_INVALID_ARG
    assert dec(p=-1) == _lib.ERR_INVALID_ARG
    assert dec(w=None) == _lib.ERR_WORKSPACE
    assert dec(wb=16) == _lib.ERR_WORKSPACE
    assert dec(scale=float("nan")) == _lib.ERR_INVALID_ARG
    assert dec(out=FAKE + 8) == _lib.ERR_ALIGNMENT


def test_decode_noalloc_argument_errors(L):
    """The no-allocation decode call makes the checks of tbq4_attn_decode, with
    the library's static scratch array standing for the workspace: partial
    states larger than the array are a workspace error before any HIP call."""
    c = _cache(batch=4, heads=8, cap=40000)

    def dec(cache=c, q=FAKE, hq=64, n_ctx=40000, out=FAKE, odt=1, p=0):
        return L.tbq4_attn_decode_noalloc(ctypes.byref(cache) if cache is not None else None, q,
                                          0, hq, n_ctx, 1.0, out, odt, p, None)
    assert dec(cache=None) == _lib.ERR_INVALID_ARG
    assert dec(out=None) == _lib.ERR_INVALID_ARG
    assert dec(odt=2) == _lib.ERR_INVALID_ARG
    assert dec(hq=72) == _lib.ERR_UNSUPPORTED
    assert dec(n_ctx=40001) == _lib.ERR_CAPACITY
    assert dec(out=FAKE + 8) == _lib.ERR_ALIGNMENT
    # 4 x 64 query rows x 1024 splits x 520 bytes = 130 MiB > 16 MiB
    assert dec(p=1024) == _lib.ERR_WORKSPACE
    per_split = 4 * 64 * 520
    assert dec(p=_lib.NOALLOC_SCRATCH_BYTES // per_split + 1) == _lib.ERR_WORKSPACE


def test_append_at_argument_errors(L):
    """Device positions cannot be checked on the host; everything else is."""
    c = _cache(heads=2, cap=64)
    app = L.tbq4_quantize_append_at
    assert app(None, FAKE, FAKE, 0, FAKE, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(c), FAKE, FAKE, 0, None, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(c), FAKE, FAKE, 9, FAKE, 1, None) == _lib.ERR_INVALID_ARG
    assert app(ctypes.byref(c), FAKE, FAKE, 0, FAKE, 65, None) == _lib.ERR_CAPACITY
    assert app(ctypes.byref(c), FAKE, FAKE, 0, FAKE, -1, None) == _lib.ERR_CAPACITY
    assert app(ctypes.byref(c), FAKE + 4, FAKE, 0, FAKE, 1, None) == _lib.ERR_ALIGNMENT
    assert app(ctypes.byref(c), FAKE, FAKE, 0, FAKE, 0, None) == _lib.OK       # nothing to do


def test_decode_varlen_argument_errors(L):
    c = _cache(heads=2, cap=64)
    ws = 1 << 20

    def dec(lens=FAKE, max_ctx=64, hq=8, out=FAKE, odt=1, p=0, w=FAKE, wb=ws):
        return L.tbq4_attn_decode_varlen(ctypes.byref(c), FAKE, 0, hq, lens, max_ctx, 1.0, out,
                                         odt, p, w, wb, None)
    assert dec(lens=None) == _lib.ERR_INVALID_ARG
    assert dec(max_ctx=0) == _lib.ERR_CAPACITY
    assert dec(max_ctx=65) == _lib.ERR_CAPACITY
    assert dec(hq=7) == _lib.ERR_UNSUPPORTED
    assert dec(out=None) == _lib.ERR_INVALID_ARG
    assert dec(odt=2) == _lib.ERR_INVALID_ARG
    assert dec(p=2000) == _lib.ERR_INVALID_ARG
    assert dec(wb=16) == _lib.ERR_WORKSPACE
    assert dec(out=FAKE + 8) == _lib.ERR_ALIGNMENT


def test_decode_step_argument_errors(L):
    """The fused step makes the append's and the decode's checks on the host
    (pos + 1 slots attended; one more partial state per head in the
    workspace)."""
    c = _cache(heads=2, cap=64)
    need = L.tbq4_decode_step_workspace_bytes(1, 2, 8, 64, 4)
    assert need == ((1 * 8 * 5 * 130 * 4 + 255) // 256) * 256
    assert L.tbq4_decode_step_workspace_bytes(1, 2, 8, 64, 1025) == 0
    assert L.tbq4_decode_step_workspace_bytes(1, 2, 8, 0, 4) == 0

    def step(cache=c, kn=FAKE, vn=FAKE, sdt=0, pos=10, positions=None, q=FAKE, qdt=0, hq=8,
             out=FAKE, odt=1, p=4, w=FAKE, wb=need):
        return L.tbq4_decode_step(ctypes.byref(cache) if cache is not None else None, kn, vn, sdt,
                                  pos, positions, q, qdt, hq, 1.0, out, odt, p, w, wb, None)
    assert step(cache=None) == _lib.ERR_INVALID_ARG
    assert step(kn=None) == _lib.ERR_INVALID_ARG
    assert step(out=None) == _lib.ERR_INVALID_ARG
    assert step(sdt=5) == _lib.ERR_INVALID_ARG
    assert step(odt=2) == _lib.ERR_INVALID_ARG
    assert step(qdt=4) == _lib.ERR_INVALID_ARG
    assert step(pos=-1) == _lib.ERR_CAPACITY
    assert step(pos=64) == _lib.ERR_CAPACITY          # slot past the capacity
    assert step(pos=2 ** 31 - 1) == _lib.ERR_CAPACITY
    assert step(hq=7) == _lib.ERR_UNSUPPORTED
    assert step(hq=18) == _lib.ERR_UNSUPPORTED
    assert step(p=1024) == _lib.ERR_INVALID_ARG       # 1024 splits + the new token's
    assert step(p=-1) == _lib.ERR_INVALID_ARG
    assert step(w=None) == _lib.ERR_WORKSPACE
    assert step(wb=need - 256) == _lib.ERR_WORKSPACE  # the decode's size is one split short
    assert step(kn=FAKE + 4) == _lib.ERR_ALIGNMENT
    assert step(out=FAKE + 8) == _lib.ERR_ALIGNMENT
    assert step(cache=_cache(cap=60)) == _lib.ERR_ALIGNMENT
    # the timed variant makes the same checks before anything is launched
    assert L.tbq4_decode_step_timed(ctypes.byref(c), FAKE, FAKE, 0, 64, None, FAKE, 0, 8, 1.0,
                                    FAKE, 1, 4, FAKE, need, None, None,
                                    None) == _lib.ERR_CAPACITY
    assert L.tbq4_decode_step_timed(ctypes.byref(c), FAKE, FAKE, 0, 10, None, FAKE, 0, 8, 1.0,
                                    None, 1, 4, FAKE, need, None, None,
                                    None) == _lib.ERR_INVALID_ARG


def test_verify_argument_errors(L):
    c = _cache(heads=2, cap=64)
    ws = 1 << 20

    def ver(n_past=10, n_q=4, hq=16, qdt=0, odt=1, p=0, out=FAKE, wb=ws):
        return L.tbq4_attn_verify(ctypes.byref(c), FAKE, qdt, hq, n_past, n_q, 1.0, out, odt, p,
                                  FAKE, wb, None)
    assert ver(n_q=0) == _lib.ERR_UNSUPPORTED
    assert ver(n_q=5) == _lib.ERR_UNSUPPORTED
    assert ver(hq=18) == _lib.ERR_UNSUPPORTED          # group of 9
    assert ver(n_past=-1) == _lib.ERR_INVALID_ARG
    assert ver(n_past=61, n_q=4) == _lib.ERR_CAPACITY  # 65 > 64
    assert ver(qdt=3) == _lib.ERR_INVALID_ARG
    assert ver(out=None) == _lib.ERR_INVALID_ARG
    assert ver(p=1025) == _lib.ERR_INVALID_ARG
    assert ver(wb=16) == _lib.ERR_WORKSPACE
    assert ver(out=FAKE + 4) == _lib.ERR_ALIGNMENT
    # workspace size: batch * n_q * n_q_heads * P * 130 * 4, rounded to 256
    assert L.tbq4_verify_workspace_bytes(1, 2, 16, 10, 4, 3) == ((1 * 4 * 16 * 3 * 520 + 255) // 256) * 256
    assert L.tbq4_verify_workspace_bytes(1, 2, 16, 10, 5, 3) == 0


def test_prefill_argument_errors(L):
    c = _cache(heads=2, cap=64)

    def pre(cache=c, q=FAKE, qdt=0, hq=16, n_past=10, n_q=4, out=FAKE, odt=1):
        return L.tbq4_attn_prefill_chunk(ctypes.byref(cache), q, qdt, hq, n_past, n_q, 0.1, out,
                                         odt, None)
    assert pre(hq=6) == _lib.ERR_UNSUPPORTED            # group of 3
    assert pre(n_past=60, n_q=5) == _lib.ERR_CAPACITY
    assert pre(n_q=0) == _lib.ERR_CAPACITY
    assert pre(n_past=-1) == _lib.ERR_CAPACITY
    assert pre(q=None) == _lib.ERR_INVALID_ARG
    assert pre(cache=_cache(head_dim=256)) == _lib.ERR_UNSUPPORTED


def test_quantize_blocks_argument_errors(L):
    q = L.tbq4_quantize_blocks
    assert q(FAKE, 0, -1, 0, FAKE, None) == _lib.ERR_INVALID_ARG
    assert q(FAKE, 5, 1, 0, FAKE, None) == _lib.ERR_INVALID_ARG
    assert q(None, 0, 1, 0, FAKE, None) == _lib.ERR_INVALID_ARG
    assert q(FAKE, 0, 0, 0, None, None) == _lib.OK


def test_mixed_format_row_bytes_and_argument_errors(L):
    assert L.tbq4_format_row_bytes(0) == o.BLOCK_BYTES == 66        # TBQ4
    assert L.tbq4_format_row_bytes(1) == 2 * o.HEAD_DIM             # binary16 rows
    assert L.tbq4_format_row_bytes(2) == o.BLOCK_BYTES3 == 50       # TBQ3
    assert L.tbq4_format_row_bytes(3) == o.Q8_ROW_BYTES == 136       # q8_0
    assert L.tbq4_format_row_bytes(4) == 0 and L.tbq4_format_row_bytes(-1) == 0

    def mc(kf=0, vf=2, cap=64, head_dim=128):
        return _lib.MixedCache(FAKE, FAKE, kf, vf, 1, 2, head_dim, cap, 0)
    app = L.tbq4_mixed_append
    assert app(ctypes.byref(mc(vf=4)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_UNSUPPORTED
    assert app(ctypes.byref(mc(kf=-1)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_UNSUPPORTED
    assert app(ctypes.byref(mc(cap=60)), FAKE, FAKE, 0, 0, 1, None) == _lib.ERR_ALIGNMENT
    assert app(ctypes.byref(mc()), FAKE, FAKE, 0, 60, 5, None) == _lib.ERR_CAPACITY
    assert app(ctypes.byref(mc()), FAKE, FAKE, 0, 0, 0, None) == _lib.OK
    ws = 1 << 20

    def dec(cache, hq=8, n_ctx=10):
        return L.tbq4_mixed_attn_decode(ctypes.byref(cache), FAKE, 0, hq, n_ctx, 0.1, FAKE, 1, 0,
                                        FAKE, ws, None)
    assert dec(mc(kf=2, vf=4)) == _lib.ERR_UNSUPPORTED
    assert dec(mc(kf=3, vf=0), n_ctx=65) == _lib.ERR_CAPACITY
    assert dec(mc(kf=2, vf=2), n_ctx=65) == _lib.ERR_CAPACITY
    assert dec(mc(kf=2, vf=1), hq=18) == _lib.ERR_UNSUPPORTED

    def pre(cache, hq=8, n_past=10, n_q=5):
        return L.tbq4_mixed_attn_prefill_chunk(ctypes.byref(cache), FAKE, 0, hq, n_past, n_q, 0.1,
                                               FAKE, 1, None)
    # q8_0 tensors are accepted: these stop at the capacity check instead
    assert pre(mc(kf=3, vf=0), n_past=60, n_q=5) == _lib.ERR_CAPACITY
    assert pre(mc(kf=0, vf=3), n_past=60, n_q=5) == _lib.ERR_CAPACITY
    assert pre(mc(kf=2, vf=4)) == _lib.ERR_UNSUPPORTED
    assert pre(mc(kf=2, vf=1), n_past=60, n_q=5) == _lib.ERR_CAPACITY
    assert pre(mc(kf=1, vf=2), hq=6) == _lib.ERR_UNSUPPORTED   # G = 3
    assert pre(mc(kf=1, vf=1), n_q=0) == _lib.ERR_CAPACITY

    def ver(cache, hq=8, n_past=10, n_q=3, p=0, wb=ws):
        return L.tbq4_mixed_attn_verify(ctypes.byref(cache), FAKE, 0, hq, n_past, n_q, 0.1, FAKE,
                                        1, p, FAKE, wb, None)
    # q8_0 tensors are accepted: these stop at the workspace check instead
    assert ver(mc(kf=3, vf=0), wb=16) == _lib.ERR_WORKSPACE
    assert ver(mc(kf=1, vf=3), wb=16) == _lib.ERR_WORKSPACE
    assert ver(mc(kf=4, vf=1)) == _lib.ERR_UNSUPPORTED
    assert ver(mc(kf=2, vf=1), n_past=62, n_q=3) == _lib.ERR_CAPACITY
    assert ver(mc(kf=1, vf=2), n_q=5) == _lib.ERR_UNSUPPORTED
    assert ver(mc(kf=2, vf=2), hq=18) == _lib.ERR_UNSUPPORTED  # G = 9
    assert ver(mc(kf=1, vf=1), wb=16) == _lib.ERR_WORKSPACE
    assert ver(mc(kf=2, vf=0), p=1025) == _lib.ERR_INVALID_ARG
