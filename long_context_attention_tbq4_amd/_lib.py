"""ctypes view of libtbq4.so (the C ABI in include/tbq4.h).

Loading fails loudly: there is no fallback implementation anywhere in this
package.  Build the library with ``python -m long_context_attention_tbq4_amd.build``.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtbq4.so")

HEAD_DIM = 128
BLOCK_BYTES = 66
MAX_SPLITS = 1024

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_ALIGNMENT, ERR_WORKSPACE, ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
F32, F16, BF16 = 0, 1, 2

EXPORTS = (
    "tbq4_cache_bytes", "tbq4_decode_auto_splits", "tbq4_decode_workspace_bytes",
    "tbq4_sign_vector", "tbq4_quantize_append", "tbq4_quantize_blocks", "tbq4_attn_decode",
    "tbq4_attn_decode_partial", "tbq4_attn_decode_partial_timed", "tbq4_attn_decode_merge",
    "tbq4_attn_prefill_chunk", "tbq4_quantize_append_at", "tbq4_attn_decode_varlen",
    "tbq4_verify_workspace_bytes", "tbq4_attn_verify", "tbq4_format_row_bytes",
    "tbq4_mixed_append", "tbq4_mixed_attn_decode", "tbq4_mixed_attn_prefill_chunk",
    "tbq4_mixed_attn_verify", "tbq4_attn_decode_noalloc",
    "tbq4_decode_step_workspace_bytes", "tbq4_decode_step", "tbq4_decode_step_timed",
    "tbq4_status_str", "tbq4_version",
)
NOALLOC_SCRATCH_BYTES = 16 << 20
# measurement helpers (include/tbq4_bench.h)
BENCH_EXPORTS = ("tbq4_bench_stream_read", "tbq4_bench_mfma_f16")


class Cache(ctypes.Structure):
    """Mirror of ``tbq4_cache``."""
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("sign_seed", ctypes.c_uint64),
    ]


class MixedCache(ctypes.Structure):
    """Mirror of ``tbq4_mixed_cache``."""
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_format", ctypes.c_int32),
        ("v_format", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("sign_seed", ctypes.c_uint64),
    ]


_lib = None


def lib():
    """The loaded library (loaded once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m long_context_attention_tbq4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
    f32, pc = ctypes.c_float, ctypes.POINTER(Cache)
    L.tbq4_cache_bytes.argtypes = [i32, i32, i32]
    L.tbq4_cache_bytes.restype = sz
    L.tbq4_decode_auto_splits.argtypes = [i32, i32, i32]
    L.tbq4_decode_auto_splits.restype = i32
    L.tbq4_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.tbq4_decode_workspace_bytes.restype = sz
    L.tbq4_sign_vector.argtypes = [u64, ctypes.POINTER(ctypes.c_uint8)]
    L.tbq4_sign_vector.restype = i32
    L.tbq4_quantize_append.argtypes = [pc, vp, vp, i32, i32, i32, vp]
    L.tbq4_quantize_append.restype = i32
    L.tbq4_quantize_blocks.argtypes = [vp, i32, i64, u64, vp, vp]
    L.tbq4_quantize_blocks.restype = i32
    L.tbq4_attn_decode.argtypes = [pc, vp, i32, i32, i32, f32, vp, i32, i32, vp, sz, vp]
    L.tbq4_attn_decode.restype = i32
    L.tbq4_attn_decode_noalloc.argtypes = [pc, vp, i32, i32, i32, f32, vp, i32, i32, vp]
    L.tbq4_attn_decode_noalloc.restype = i32
    L.tbq4_attn_decode_partial.argtypes = [pc, vp, i32, i32, i32, f32, i32,
                                           ctypes.POINTER(i32), vp, sz, vp]
    L.tbq4_attn_decode_partial.restype = i32
    L.tbq4_attn_decode_partial_timed.argtypes = [pc, vp, i32, i32, i32, f32, i32,
                                                 ctypes.POINTER(i32), vp, sz, vp, vp, vp]
    L.tbq4_attn_decode_partial_timed.restype = i32
    L.tbq4_attn_decode_merge.argtypes = [vp, sz, i32, i32, i32, u64, vp, i32, vp]
    L.tbq4_attn_decode_merge.restype = i32
    L.tbq4_quantize_append_at.argtypes = [pc, vp, vp, i32, vp, i32, vp]
    L.tbq4_quantize_append_at.restype = i32
    L.tbq4_attn_decode_varlen.argtypes = [pc, vp, i32, i32, vp, i32, f32, vp, i32, i32, vp, sz, vp]
    L.tbq4_attn_decode_varlen.restype = i32
    L.tbq4_decode_step_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.tbq4_decode_step_workspace_bytes.restype = sz
    L.tbq4_decode_step.argtypes = [pc, vp, vp, i32, i32, vp, vp, i32, i32, f32, vp, i32, i32, vp,
                                   sz, vp]
    L.tbq4_decode_step.restype = i32
    L.tbq4_decode_step_timed.argtypes = [pc, vp, vp, i32, i32, vp, vp, i32, i32, f32, vp, i32,
                                         i32, vp, sz, vp, vp, vp]
    L.tbq4_decode_step_timed.restype = i32
    L.tbq4_verify_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.tbq4_verify_workspace_bytes.restype = sz
    L.tbq4_attn_verify.argtypes = [pc, vp, i32, i32, i32, i32, f32, vp, i32, i32, vp, sz, vp]
    L.tbq4_attn_verify.restype = i32
    pm = ctypes.POINTER(MixedCache)
    L.tbq4_format_row_bytes.argtypes = [i32]
    L.tbq4_format_row_bytes.restype = sz
    L.tbq4_mixed_append.argtypes = [pm, vp, vp, i32, i32, i32, vp]
    L.tbq4_mixed_append.restype = i32
    L.tbq4_mixed_attn_decode.argtypes = [pm, vp, i32, i32, i32, f32, vp, i32, i32, vp, sz, vp]
    L.tbq4_mixed_attn_decode.restype = i32
    L.tbq4_mixed_attn_prefill_chunk.argtypes = [pm, vp, i32, i32, i32, i32, f32, vp, i32, vp]
    L.tbq4_mixed_attn_prefill_chunk.restype = i32
    L.tbq4_mixed_attn_verify.argtypes = [pm, vp, i32, i32, i32, i32, f32, vp, i32, i32, vp, sz, vp]
    L.tbq4_mixed_attn_verify.restype = i32
    L.tbq4_attn_prefill_chunk.argtypes = [pc, vp, i32, i32, i32, i32, f32, vp, i32, vp]
    L.tbq4_attn_prefill_chunk.restype = i32
    L.tbq4_bench_stream_read.argtypes = [vp, sz, vp, i32, vp]
    L.tbq4_bench_stream_read.restype = i32
    L.tbq4_bench_mfma_f16.argtypes = [i32, vp, i32, vp]
    L.tbq4_bench_mfma_f16.restype = i32
    L.tbq4_status_str.argtypes = [i32]
    L.tbq4_status_str.restype = ctypes.c_char_p
    L.tbq4_version.argtypes = []
    L.tbq4_version.restype = ctypes.c_char_p
    _lib = L
    return L
