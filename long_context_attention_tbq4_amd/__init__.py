"""TBQ4 fused long-context attention for AMD Instinct MI355X (gfx950).

Python binding of libtbq4.so: argument marshalling only.  Every step of the
hot path -- quantise-append, split-K decode attention, prefill-chunk
attention -- runs in the library's HIP kernels; torch supplies device memory
and the current stream.

Method: page "Kontekst 262K na jednej RTX 4090: co dodałem do
llama.cpp-turboq", section "Od czego zacząłem" -- flash attention reads raw
TBQ4 blocks (128 values in 66 bytes: 2-byte scale + 64 bytes of 4-bit
indices) and dequantises them in its inner loop, in the rotated Hadamard
domain, with no dequantisation pass and no F16 buffer.
"""

import ctypes

import torch

from . import _lib
from ._lib import BLOCK_BYTES, HEAD_DIM, MAX_SPLITS, NOALLOC_SCRATCH_BYTES

__all__ = [
    "TBQ4Error", "KVCache", "quantize_append", "quantize_blocks", "attn_decode",
    "attn_decode_partial", "attn_decode_merge", "attn_decode_noalloc", "quantize_append_at",
    "attn_decode_varlen", "NOALLOC_SCRATCH_BYTES", "decode_step", "decode_step_workspace_bytes",
    "attn_verify", "verify_workspace_bytes", "MixedKVCache", "mixed_append",
    "mixed_attn_decode", "mixed_attn_prefill_chunk", "mixed_attn_verify", "FMT_TBQ4", "FMT_F16", "FMT_TBQ3", "FMT_Q8_0",
    "attn_prefill_chunk", "sign_vector", "cache_bytes", "decode_auto_splits",
    "decode_workspace_bytes", "version", "HEAD_DIM", "BLOCK_BYTES", "MAX_SPLITS",
]

_DT = {torch.float32: _lib.F32, torch.float16: _lib.F16, torch.bfloat16: _lib.BF16}


class TBQ4Error(RuntimeError):
    def __init__(self, status, what):
        msg = _lib.lib().tbq4_status_str(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def _check(status, what):
    if status != _lib.OK:
        raise TBQ4Error(status, what)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _dtype(t):
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _require(t, name, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class KVCache:
    """One layer's TBQ4 K and V caches: uint8 device tensors of shape
    [batch][n_kv_heads][capacity][66] (head-major rows of 66-byte blocks)."""

    def __init__(self, batch, n_kv_heads, capacity, sign_seed=0, device="cuda"):
        if capacity % 8:
            raise ValueError("capacity must be a multiple of 8")
        shape = (batch, n_kv_heads, capacity, BLOCK_BYTES)
        self.k = torch.zeros(shape, dtype=torch.uint8, device=device)
        self.v = torch.zeros(shape, dtype=torch.uint8, device=device)
        self.batch, self.n_kv_heads, self.capacity = batch, n_kv_heads, capacity
        self.sign_seed = sign_seed

    @property
    def device(self):
        return self.k.device

    def descriptor(self):
        return _lib.Cache(self.k.data_ptr(), self.v.data_ptr(), self.batch, self.n_kv_heads,
                          HEAD_DIM, self.capacity, self.sign_seed)


FMT_TBQ4, FMT_F16, FMT_TBQ3, FMT_Q8_0 = 0, 1, 2, 3
_ROW_BYTES = {FMT_TBQ4: BLOCK_BYTES, FMT_F16: 2 * HEAD_DIM, FMT_TBQ3: 50, FMT_Q8_0: 136}


class MixedKVCache:
    """One layer's K and V caches, each in its own format: FMT_TBQ4 (uint8
    [batch][n_kv_heads][capacity][66]), FMT_TBQ3 (uint8 [...][50]: binary16
    scale + 128 3-bit codes), FMT_Q8_0 (uint8 [...][136]: four blocks of a
    binary16 scale + 32 int8 codes, not rotated) or FMT_F16 (uint8 view of
    fp16 [batch][n_kv_heads][capacity][128], not rotated)."""

    def __init__(self, batch, n_kv_heads, capacity, k_format, v_format, sign_seed=0,
                 device="cuda"):
        if capacity % 8:
            raise ValueError("capacity must be a multiple of 8")
        if k_format not in _ROW_BYTES or v_format not in _ROW_BYTES:
            raise ValueError("unknown cache format")
        self.k = torch.zeros((batch, n_kv_heads, capacity, _ROW_BYTES[k_format]), dtype=torch.uint8,
                             device=device)
        self.v = torch.zeros((batch, n_kv_heads, capacity, _ROW_BYTES[v_format]), dtype=torch.uint8,
                             device=device)
        self.k_format, self.v_format = k_format, v_format
        self.batch, self.n_kv_heads, self.capacity = batch, n_kv_heads, capacity
        self.sign_seed = sign_seed

    @property
    def device(self):
        return self.k.device

    def descriptor(self):
        return _lib.MixedCache(self.k.data_ptr(), self.v.data_ptr(), self.k_format, self.v_format,
                               self.batch, self.n_kv_heads, HEAD_DIM, self.capacity, self.sign_seed)


def mixed_append(cache, k_new, v_new, pos):
    """Append k_new, v_new ([batch][n_new][n_kv_heads][128]) into slots
    [pos, pos + n_new), each tensor in its cache's format."""
    _require(k_new, "k_new")
    _require(v_new, "v_new", k_new.shape)
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    B, n_new, H, D = k_new.shape
    if (B, H, D) != (cache.batch, cache.n_kv_heads, HEAD_DIM):
        raise ValueError("k_new shape does not match the cache")
    d = cache.descriptor()
    _check(_lib.lib().tbq4_mixed_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _dtype(k_new),
                                        pos, n_new, _stream(cache.device)), "tbq4_mixed_append")


def mixed_attn_decode(cache, q, n_ctx, softmax_scale, n_splits=0, out=None,
                      out_dtype=torch.float16, workspace=None):
    """Decode attention over a MixedKVCache; same shapes as attn_decode."""
    _require(q, "q")
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, Hq, D))
    need = decode_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, n_ctx, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    d = cache.descriptor()
    _check(_lib.lib().tbq4_mixed_attn_decode(
        ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_ctx, float(softmax_scale), _ptr(out),
        _dtype(out), n_splits, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device)), "tbq4_mixed_attn_decode")
    return out


def mixed_attn_prefill_chunk(cache, q, n_past, softmax_scale, out=None, out_dtype=torch.float16):
    """Causal prefill-chunk attention over a MixedKVCache whose K and V are
    TBQ4, TBQ3, q8_0 or fp16; same shapes as attn_prefill_chunk."""
    _require(q, "q")
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, n_q, Hq, D))
    d = cache.descriptor()
    _check(_lib.lib().tbq4_mixed_attn_prefill_chunk(
        ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_past, n_q, float(softmax_scale), _ptr(out),
        _dtype(out), _stream(q.device)), "tbq4_mixed_attn_prefill_chunk")
    return out


def mixed_attn_verify(cache, q, n_past, softmax_scale, n_splits=0, out=None,
                      out_dtype=torch.float16, workspace=None):
    """Multi-query verify attention over a MixedKVCache whose K and V are
    TBQ4, TBQ3, q8_0 or fp16; same shapes as attn_verify."""
    _require(q, "q")
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, n_q, Hq, D))
    need = verify_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, n_past, n_q, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    d = cache.descriptor()
    _check(_lib.lib().tbq4_mixed_attn_verify(
        ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_past, n_q, float(softmax_scale), _ptr(out),
        _dtype(out), n_splits, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device)), "tbq4_mixed_attn_verify")
    return out


def quantize_append(cache, k_new, v_new, pos):
    """Quantise k_new, v_new ([batch][n_new][n_kv_heads][128], fp32/fp16/bf16)
    into token slots [pos, pos + n_new) of every sequence."""
    _require(k_new, "k_new")
    _require(v_new, "v_new", k_new.shape)
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    B, n_new, H, D = k_new.shape
    if (B, H, D) != (cache.batch, cache.n_kv_heads, HEAD_DIM):
        raise ValueError("k_new shape does not match the cache")
    d = cache.descriptor()
    _check(_lib.lib().tbq4_quantize_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new),
                                           _dtype(k_new), pos, n_new, _stream(cache.device)),
           "tbq4_quantize_append")


def quantize_append_at(cache, k_new, v_new, positions):
    """As quantize_append, but sequence b writes slots [positions[b],
    positions[b] + n_new); positions is a device int32 tensor [batch], read
    when the kernel runs (graph-capturable).  Slots outside the capacity are
    skipped."""
    _require(k_new, "k_new")
    _require(v_new, "v_new", k_new.shape)
    _require(positions, "positions", (cache.batch,))
    if positions.dtype != torch.int32:
        raise TypeError("positions must be int32")
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    B, n_new, H, D = k_new.shape
    if (B, H, D) != (cache.batch, cache.n_kv_heads, HEAD_DIM):
        raise ValueError("k_new shape does not match the cache")
    d = cache.descriptor()
    _check(_lib.lib().tbq4_quantize_append_at(ctypes.byref(d), _ptr(k_new), _ptr(v_new),
                                              _dtype(k_new), _ptr(positions), n_new,
                                              _stream(cache.device)),
           "tbq4_quantize_append_at")


def attn_decode_varlen(cache, q, ctx_lens, max_ctx, softmax_scale, n_splits=0, out=None,
                       out_dtype=torch.float16, workspace=None):
    """Decode attention where sequence b attends slots [0, ctx_lens[b]);
    ctx_lens is a device int32 tensor [batch] (clamped to [0, max_ctx]) read
    when the kernel runs, so a captured graph stays valid as it changes."""
    _require(q, "q")
    B, Hq, D = q.shape
    _require(ctx_lens, "ctx_lens", (cache.batch,))
    if ctx_lens.dtype != torch.int32:
        raise TypeError("ctx_lens must be int32")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, Hq, D))
    need = decode_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, max_ctx, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    d = cache.descriptor()
    _check(_lib.lib().tbq4_attn_decode_varlen(
        ctypes.byref(d), _ptr(q), _dtype(q), Hq, _ptr(ctx_lens), max_ctx, float(softmax_scale),
        _ptr(out), _dtype(out), n_splits, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device)),
        "tbq4_attn_decode_varlen")
    return out


def decode_step_workspace_bytes(batch, n_kv_heads, n_q_heads, n_ctx, n_splits=0):
    return _lib.lib().tbq4_decode_step_workspace_bytes(batch, n_kv_heads, n_q_heads, n_ctx,
                                                       n_splits)


def decode_step(cache, k_new, v_new, q, pos, softmax_scale, positions=None, n_splits=0, out=None,
                out_dtype=torch.float16, workspace=None, events=None):
    """Append one token per sequence (k_new, v_new: [batch][1][n_kv_heads][128])
    and attend over the cache that holds it, in one decode launch and the
    merge.  positions=None: every sequence writes slot pos and attends
    [0, pos]; else positions is a device int32 tensor [batch] read when the
    kernel runs (sequence b writes slot positions[b] and attends
    [0, positions[b]]) and pos bounds them.  events: optional (start, stop)
    hipEvent_t handles that the split kernel's dispatch records.  Returns out
    [batch][n_q_heads][128]."""
    _require(q, "q")
    _require(k_new, "k_new")
    _require(v_new, "v_new", k_new.shape)
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    if tuple(k_new.shape) != (cache.batch, 1, cache.n_kv_heads, HEAD_DIM):
        raise ValueError("k_new must be [batch][1][n_kv_heads][128]")
    if positions is not None:
        _require(positions, "positions", (cache.batch,))
        if positions.dtype != torch.int32:
            raise TypeError("positions must be int32")
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, Hq, D))
    if workspace is None:
        need = decode_step_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, pos + 1, n_splits)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    d = cache.descriptor()
    args = (ctypes.byref(d), _ptr(k_new), _ptr(v_new), _dtype(k_new), pos,
            _ptr(positions) if positions is not None else None, _ptr(q), _dtype(q), Hq,
            float(softmax_scale), _ptr(out), _dtype(out), n_splits, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    if events is None:
        _check(_lib.lib().tbq4_decode_step(*args), "tbq4_decode_step")
    else:
        _check(_lib.lib().tbq4_decode_step_timed(*args, ctypes.c_void_p(events[0]),
                                                 ctypes.c_void_p(events[1])),
               "tbq4_decode_step_timed")
    return out


def verify_workspace_bytes(batch, n_kv_heads, n_q_heads, n_past, n_q, n_splits=0):
    return _lib.lib().tbq4_verify_workspace_bytes(batch, n_kv_heads, n_q_heads, n_past, n_q,
                                                  n_splits)


def attn_verify(cache, q, n_past, softmax_scale, n_splits=0, out=None, out_dtype=torch.float16,
                workspace=None):
    """Multi-query verify attention: q [batch][n_q][n_q_heads][128] with
    n_q <= 4; query i attends slots [0, n_past + i].  Returns out
    ([batch][n_q][n_q_heads][128])."""
    _require(q, "q")
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, n_q, Hq, D))
    need = verify_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, n_past, n_q, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    d = cache.descriptor()
    _check(_lib.lib().tbq4_attn_verify(ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_past, n_q,
                                       float(softmax_scale), _ptr(out), _dtype(out), n_splits,
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(q.device)), "tbq4_attn_verify")
    return out


def quantize_blocks(x, sign_seed=0, out=None):
    """Quantise a contiguous (..., 128) tensor into (..., 66) uint8 blocks."""
    _require(x, "x")
    if x.shape[-1] != HEAD_DIM:
        raise ValueError("last dimension must be 128")
    n = x.numel() // HEAD_DIM
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (BLOCK_BYTES,), dtype=torch.uint8, device=x.device)
    _require(out, "out", tuple(x.shape[:-1]) + (BLOCK_BYTES,))
    _check(_lib.lib().tbq4_quantize_blocks(_ptr(x), _dtype(x), n, sign_seed, _ptr(out),
                                           _stream(x.device)), "tbq4_quantize_blocks")
    return out


def decode_auto_splits(batch, n_kv_heads, n_ctx):
    return _lib.lib().tbq4_decode_auto_splits(batch, n_kv_heads, n_ctx)


def decode_workspace_bytes(batch, n_kv_heads, n_q_heads, n_ctx, n_splits=0):
    return _lib.lib().tbq4_decode_workspace_bytes(batch, n_kv_heads, n_q_heads, n_ctx, n_splits)


def attn_decode(cache, q, n_ctx, softmax_scale, n_splits=0, out=None, out_dtype=torch.float16,
                workspace=None):
    """Decode attention of q ([batch][n_q_heads][128], fp32/fp16/bf16) against
    cached slots [0, n_ctx).  Returns out ([batch][n_q_heads][128])."""
    _require(q, "q")
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, Hq, D))
    need = decode_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, n_ctx, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    d = cache.descriptor()
    _check(_lib.lib().tbq4_attn_decode(ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_ctx,
                                       float(softmax_scale), _ptr(out), _dtype(out), n_splits,
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(q.device)), "tbq4_attn_decode")
    return out


def attn_decode_noalloc(cache, q, n_ctx, softmax_scale, n_splits=0, out=None,
                        out_dtype=torch.float16):
    """attn_decode without a workspace: the library's static per-device
    scratch array holds the split-K partial states (nothing is allocated by
    the call itself; pass ``out`` to allocate nothing at all).  Calls that
    overlap on one device race; partial states larger than
    NOALLOC_SCRATCH_BYTES raise TBQ4Error (workspace)."""
    _require(q, "q")
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, Hq, D))
    d = cache.descriptor()
    _check(_lib.lib().tbq4_attn_decode_noalloc(ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_ctx,
                                               float(softmax_scale), _ptr(out), _dtype(out),
                                               n_splits, _stream(q.device)),
           "tbq4_attn_decode_noalloc")
    return out


def attn_decode_partial(cache, q, n_ctx, softmax_scale, n_splits=0, workspace=None,
                        events=None):
    """First decode phase: per-split partial softmax states into `workspace`
    (layout in include/tbq4.h).  Returns (workspace, n_splits_used).

    ``events``: optional (start, stop) raw hipEvent_t handles (ints); the split
    kernel's dispatch records them at its start and end."""
    _require(q, "q")
    B, Hq, D = q.shape
    need = decode_workspace_bytes(cache.batch, cache.n_kv_heads, Hq, n_ctx, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    used = ctypes.c_int32(0)
    d = cache.descriptor()
    nbytes = workspace.numel() * workspace.element_size()
    if events is None:
        _check(_lib.lib().tbq4_attn_decode_partial(
            ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_ctx, float(softmax_scale), n_splits,
            ctypes.byref(used), _ptr(workspace), nbytes, _stream(q.device)),
            "tbq4_attn_decode_partial")
    else:
        _check(_lib.lib().tbq4_attn_decode_partial_timed(
            ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_ctx, float(softmax_scale), n_splits,
            ctypes.byref(used), _ptr(workspace), nbytes, _stream(q.device),
            ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1])),
            "tbq4_attn_decode_partial_timed")
    return workspace, used.value


def attn_decode_merge(workspace, batch, n_q_heads, n_splits, sign_seed=0, out=None,
                      out_dtype=torch.float16):
    """Second decode phase: merge `n_splits` partial states per (sequence,
    head), normalise and rotate back.  Returns out ([batch][n_q_heads][128])."""
    if out is None:
        out = torch.empty((batch, n_q_heads, HEAD_DIM), dtype=out_dtype, device=workspace.device)
    _require(out, "out", (batch, n_q_heads, HEAD_DIM))
    _check(_lib.lib().tbq4_attn_decode_merge(
        _ptr(workspace), workspace.numel() * workspace.element_size(), batch, n_q_heads, n_splits,
        sign_seed, _ptr(out), _dtype(out), _stream(out.device)), "tbq4_attn_decode_merge")
    return out


def attn_prefill_chunk(cache, q, n_past, softmax_scale, out=None, out_dtype=torch.float16):
    """Causal prefill-chunk attention of q ([batch][n_q][n_q_heads][128]):
    query i attends slots [0, n_past + i]."""
    _require(q, "q")
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    _require(out, "out", (B, n_q, Hq, D))
    d = cache.descriptor()
    _check(_lib.lib().tbq4_attn_prefill_chunk(ctypes.byref(d), _ptr(q), _dtype(q), Hq, n_past,
                                              n_q, float(softmax_scale), _ptr(out), _dtype(out),
                                              _stream(q.device)), "tbq4_attn_prefill_chunk")
    return out


def sign_vector(seed):
    """The 16 sign bytes for ``seed`` (bit i set means s_i = -1)."""
    buf = (ctypes.c_uint8 * 16)()
    _check(_lib.lib().tbq4_sign_vector(seed, buf), "tbq4_sign_vector")
    return bytes(buf)


def cache_bytes(batch, n_kv_heads, capacity):
    return _lib.lib().tbq4_cache_bytes(batch, n_kv_heads, capacity)


def version():
    return _lib.lib().tbq4_version().decode()
