"""Seeded generators (see the package docstring for the recipes)."""

from dataclasses import dataclass
import math
import os

import numpy as np

K, V, Q = 0, 1, 2                 # tensor ids used in the stream keys
_BULK, _PICK, _CSCALE, _DRIFT, _QUERY = 0, 1, 2, 3, 4
CHUNK = 16384                     # tokens per independently seeded chunk
D = 128


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    n_ctx: int                    # cached tokens (decode) / n_past (prefill)
    kind: str                     # value recipe
    softmax_scale: float
    q_scale: float = 1.0          # Q is drawn as q_scale * N(0,1)
    n_q: int = 0                  # prefill chunk length
    layers: int = 1
    steps: int = 0                # long-decode steps


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 4, 1024, "tiny", 1.0 / math.sqrt(128)),
    "decode16k": Workload("decode16k", 1, 1, 8, 64, 16384, "gauss_outlier", 1.0,
                          q_scale=1.0 / math.sqrt(128)),
    "decode96k": Workload("decode96k", 2, 4, 8, 64, 98304, "student_scaled",
                          1.0 / math.sqrt(128)),
    "decode128k": Workload("decode128k", 2, 4, 8, 64, 131072, "student_scaled",
                           1.0 / math.sqrt(128)),
    "prefill": Workload("prefill", 3, 1, 8, 64, 131072, "gauss_outlier",
                        1.0 / math.sqrt(128), n_q=2048),
    "longdecode": Workload("longdecode", 4, 1, 8, 64, 262080, "student_drift",
                           1.0 / math.sqrt(128), layers=4, steps=64),
}


def _rng(*key):
    return np.random.default_rng([0] + [int(k) for k in key])


# --------------------------------------------------------------------------
# tiny: one default_rng(0) stream, drawn in the order K, V, Q, outlier channel
# --------------------------------------------------------------------------
def tiny_inputs():
    """Returns (k, v, q, channel): k, v fp32 (1, 1024, 1, 128) in the
    [batch][token][kv head][dim] layout, q fp32 (1, 4, 128)."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1024, 1, D))
    v = rng.standard_normal((1024, 1, D))
    q = rng.standard_normal((1, 4, D))
    c = int(rng.integers(D))
    k[:, :, c] *= 20.0
    return (k[None].astype(np.float32), v[None].astype(np.float32),
            q.astype(np.float32), c)


# --------------------------------------------------------------------------
# bulk K/V rows for one (layer, tensor, sequence, KV head)
# --------------------------------------------------------------------------
def _outlier_channels(w, layer, tensor, g):
    return _rng(w.cfg_id, layer, tensor, _PICK, g).choice(D, size=2, replace=False)


def _channel_scales(w, layer, tensor):
    return _rng(w.cfg_id, layer, tensor, _CSCALE).uniform(0.5, 4.0, size=(w.n_kv_heads, D))


def _chunk(w, layer, tensor, b, g, c):
    """fp64 values of chunk c (tokens c*CHUNK ... c*CHUNK+CHUNK-1) before any
    per-position drift."""
    r = _rng(w.cfg_id, layer, tensor, _BULK, b, g, c)
    if w.kind == "gauss_outlier":
        x = r.standard_normal((CHUNK, D))
        x[:, _outlier_channels(w, layer, tensor, g)] *= 15.0
    elif w.kind == "student_scaled":
        x = r.standard_t(5, size=(CHUNK, D)) * _channel_scales(w, layer, tensor)[g]
    elif w.kind == "student_drift":
        x = r.standard_t(3, size=(CHUNK, D))
    else:
        raise ValueError(w.kind)
    return x


def _drift_steps(w, layer, tensor, b, g, c):
    return _rng(w.cfg_id, layer, tensor, _DRIFT, b, g, c).normal(0.0, 0.01, size=(CHUNK, D))


def kv_rows(w, layer, tensor, b, g, t0, t1):
    """fp32 array (t1 - t0, 128): K (tensor=0) or V (tensor=1) rows of sequence
    b, KV head g, at positions t0 .. t1-1."""
    if w.kind == "tiny":
        k, v, _, _ = tiny_inputs()
        return (k if tensor == K else v)[b, t0:t1, g].copy()
    out = np.empty((t1 - t0, D), dtype=np.float32)
    if t1 <= t0:
        return out
    c0, c1 = t0 // CHUNK, (t1 - 1) // CHUNK
    mu = np.zeros(D)
    if w.kind == "student_drift":
        for c in range(c0):                       # walk state at chunk c0
            mu = mu + _drift_steps(w, layer, tensor, b, g, c).sum(axis=0)
    for c in range(c0, c1 + 1):
        x = _chunk(w, layer, tensor, b, g, c)
        if w.kind == "student_drift":
            walk = mu + np.cumsum(_drift_steps(w, layer, tensor, b, g, c), axis=0)
            mu = walk[-1]
            x = x + walk
        a = max(t0, c * CHUNK)
        e = min(t1, (c + 1) * CHUNK)
        out[a - t0:e - t0] = x[a - c * CHUNK:e - c * CHUNK]
    return out


def _rows_job(args):
    w, layer, tensor, b, g, t0, t1 = args
    return kv_rows(w, layer, tensor, b, g, t0, t1)


def kv_tensor(w, layer, tensor, t0, t1, workers=None):
    """fp32 (B, t1 - t0, H_kv, 128) in the [batch][token][kv head][dim] layout
    the append call takes.  (b, g) slices are drawn in parallel processes."""
    B, H = w.batch, w.n_kv_heads
    out = np.empty((B, t1 - t0, H, D), dtype=np.float32)
    jobs = [(w, layer, tensor, b, g, t0, t1) for b in range(B) for g in range(H)]
    n = workers if workers is not None else min(len(jobs), os.cpu_count() or 1, 16)
    if n <= 1 or (t1 - t0) * len(jobs) < 4 * CHUNK:
        for j in jobs:
            out[j[3], :, j[4]] = _rows_job(j)
    else:
        # worker processes are stopped by a sentinel, not a signal, so the
        # pool also shuts down cleanly under a profiler
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as ex:
            for j, rows in zip(jobs, ex.map(_rows_job, jobs)):
                out[j[3], :, j[4]] = rows
    return out


# --------------------------------------------------------------------------
# queries
# --------------------------------------------------------------------------
def q_decode(w, layer=0, step=0):
    """fp32 (B, H_q, 128): one decode query per sequence and head."""
    if w.kind == "tiny":
        return tiny_inputs()[2]
    r = _rng(w.cfg_id, layer, Q, _QUERY, step)
    return (w.q_scale * r.standard_normal((w.batch, w.n_q_heads, D))).astype(np.float32)


def q_prefill(w, layer=0, outliers=False):
    """fp32 (B, n_q, H_q, 128): the chunk's queries.  With ``outliers`` two
    channels per query head are also scaled x15 (the stress variant)."""
    r = _rng(w.cfg_id, layer, Q, _QUERY, 0)
    q = w.q_scale * r.standard_normal((w.batch, w.n_q, w.n_q_heads, D))
    if outliers:
        for h in range(w.n_q_heads):
            q[:, :, h, _outlier_channels(w, layer, Q, h)] *= 15.0
    return q.astype(np.float32)
