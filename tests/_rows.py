"""Oracle jobs for the full-size parity tests, run in worker processes.

Each job regenerates rows of a workload from their seeds (``workloads``),
quantises them with the fp64 oracle and computes the reference attention of
the requested queries on the dequantised rows.  Nothing here reads a value
produced by the GPU: the parent test compares the GPU's bytes and outputs with
what these jobs return.  (No method arithmetic lives here: every step is an
oracle call.)
"""

import os

import numpy as np

from oracle import tbq4_oracle as o
from workloads import WORKLOADS, K, V, kv_rows, q_prefill


def workers(n_jobs):
    """Worker processes for the oracle jobs: at most 16 (a GPU machine's CPU
    share), at most the CPUs this process may run on."""
    return max(1, min(n_jobs, 16, len(os.sched_getaffinity(0))))


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(2)
    except Exception:
        pass


def decode_row(args):
    """One (layer, sequence, KV head) row of a decode workload, slots
    [0, t_end): returns (K bytes, V bytes, {tag: reference}) where each
    (tag, q_rows, n, scale) of ``jobs`` asks for softmax attention of q_rows
    (G, 128) over the first n dequantised slots."""
    wname, layer, b, g, t_end, jobs = args
    _limit_blas()
    w = WORKLOADS[wname]
    kc = o.quantize_blocks(kv_rows(w, layer, K, b, g, 0, t_end))[0]
    vc = o.quantize_blocks(kv_rows(w, layer, V, b, g, 0, t_end))[0]
    Kd, Vd = o.dequantize_blocks(kc), o.dequantize_blocks(vc)
    refs = {tag: o.attn_decode_rows_ref(qr, Kd[:n], Vd[:n], sc) for tag, qr, n, sc in jobs}
    return kc, vc, refs


def prefill_group(args):
    """KV head ``g`` of the prefill workload (the cached prefix and the chunk,
    slots [0, n_past + n_q)): returns (K bytes, V bytes, {outliers: reference
    of chunk queries ``rows``, (len(rows), G, 128)}) for the plain queries and,
    when asked, the queries with outlier channels."""
    wname, g, rows, variants = args
    _limit_blas()
    w = WORKLOADS[wname]
    T = w.n_ctx + w.n_q
    G = w.n_q_heads // w.n_kv_heads
    kc = o.quantize_blocks(kv_rows(w, 0, K, 0, g, 0, T))[0]
    vc = o.quantize_blocks(kv_rows(w, 0, V, 0, g, 0, T))[0]
    Kd, Vd = o.dequantize_blocks(kc), o.dequantize_blocks(vc)
    refs = {}
    for outliers in variants:
        q = q_prefill(w, outliers=outliers)[0][:, g * G:(g + 1) * G]   # (n_q, G, 128)
        refs[outliers] = o.attn_prefill_rows_ref(q[rows], Kd, Vd, w.n_ctx, rows, w.softmax_scale)
    return kc, vc, refs


def pool_map(fn, jobs):
    """Run ``fn`` over ``jobs`` in spawned worker processes (results in order;
    a line is printed as each job ends, seen when pytest runs with -s)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    out = []
    with ProcessPoolExecutor(workers(len(jobs)), mp_context=mp.get_context("spawn")) as ex:
        for i, r in enumerate(ex.map(fn, jobs)):
            print(f"[oracle] {fn.__name__}: {i + 1}/{len(jobs)} jobs done", flush=True)
            out.append(r)
    return out


def random_rows(seed, n, k):
    """k distinct sorted indices in [0, n) from a seeded stream."""
    return np.sort(np.random.default_rng(seed).choice(n, size=k, replace=False))
