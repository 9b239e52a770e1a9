"""Benchmark of the TBQ4 attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--splits P] [--settle S]
                    [--no-prefill] [--no-cpu-baseline] [--no-formats] [--no-contexts]

One step = one pass of the whole decode hot path over the decode128k workload
(batch 4 independent sequences, 8 KV / 64 query heads, head_dim 128, 131072
cached tokens in TBQ4 K and V caches resident in HBM): quantise-append the new
token's K and V for every sequence, then split-K decode attention over all
131072 slots (partial kernel + merge kernel).  The headline value is the
step's algorithmic HBM bytes (packed K+V read, q read, output written, appended
rows) divided by the step time, in GB/s.  The prefill-chunk workload (2048
queries on 131072 cached tokens, 8 KV / 64 query heads, append of the chunk's
K/V then causal attention) is timed in the same run and reported under
"prefill" in TFLOP/s (4 * 128 * 64 FLOPs per unmasked (query, key) pair).
The same decode rows stored as TBQ3, q8_0 or fp16 K / V tensors (mixed
formats) are timed under "formats" (one decode call per format pair, KV GB/s),
and the prefill chunk over TBQ3 and fp16 caches under "prefill"."formats".
Decode at 16384 slots (batch 1) and the 4-layer long decode at 262144 slots
(batch 1, 64 append + decode steps per layer) are timed under "contexts".

Before the W warm-up steps, S untimed steps (default 1000, ~0.12 s) let the
clocks settle: the first milliseconds of sustained load run faster, then the
clocks dip and recover over tens of milliseconds.  The step value is timed
over K steps without any event markers.  A second loop of the same K steps
records HIP events from the dispatch of every decode-partial launch (start and
end of that kernel's execution; each pair of markers leaves the GPU idle for
several microseconds around the kernel, which is why the step time is taken
without them): their mean is reported as kernel_ms_in_step.  Then the split
kernel alone is launched K times back to back between two events on the
stream it runs on: its mean duration there is the roofline's kernel_ms (the
dispatch-recorded events read a few microseconds per call more than a kernel
trace of the same calls).
The CPU oracle is timed on a bounded sample of the same workload (rows of the
decode cache, fp64 dequantise + attention) on the host's cores.

Prints ONE JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "TBQ4 attn: decode HBM GB/s (% peak) @128K; prefill-chunk TFLOP/s"

# HBM bytes per decode_split_kernel launch on this workload (64 splits), from
# two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch)
# scaled by what the same counters read for a plain 256 MiB device copy
# (FETCH_SIZE reads half the copied bytes -> x2.0; WRITE_SIZE reads them all
# -> x1.0).  Reported only while the kernel's sources hash to the version the
# counters were taken on; otherwise the traffic is unknown (null).
KERNEL_SOURCES = ("decode.hip", "tbq4_device.h", "tbq4_launch.h")
TRAFFIC = {"sources_sha256": "f996f0500e8e79e3335e2961a082db29febccdb54fa0693c84bd2e5db80ad016",
           "n_splits": 64, "fetch_kib": 271200.9, "fetch_factor": 2.0,
           "write_kib": 8704.1, "write_factor": 1.0}


def measured_traffic(n_splits):
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                       "long_context_attention_tbq4_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != TRAFFIC["sources_sha256"] or n_splits != TRAFFIC["n_splits"]:
        return None
    return round(1024 * (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_factor"]
                         + TRAFFIC["write_kib"] * TRAFFIC["write_factor"]))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--settle", type=int, default=SETTLE_STEPS,
                   help="untimed decode steps before the warm-up steps (clock settling)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-contexts", action="store_true",
                   help="skip the 16K and 262K decode measurements")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-formats", dest="formats", action="store_false",
                   help="skip the decode timings of the TBQ3 / fp16 cache formats")
    p.add_argument("--prefill-steps", type=int, default=0)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB five times "
                        "(reference for the profiler's byte counters) and exit")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Timing events of the HIP runtime torch already loaded, handed to the
    library so that the kernel dispatch itself records them."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def pair(self, i):
        return self.ev[2 * i], self.ev[2 * i + 1]

    def elapsed_ms(self):
        out = []
        for i in range(len(self.ev) // 2):
            ms = self.ct.c_float()
            rc = self.rt.hipEventElapsedTime(self.ct.byref(ms), self.ev[2 * i], self.ev[2 * i + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out.append(ms.value)
        return out

    def destroy(self):
        for e in self.ev:
            self.rt.hipEventDestroy(e)
        self.ev = []


def fill_cache(tb, torch, cache, w, t0, t1, chunk=32768, keep=None):
    """Append tokens t0 .. t1 of the workload to the TBQ4 cache; with `keep`
    (a list) the fp32 K/V chunks stay resident on the GPU for later caches."""
    from workloads import K, V, kv_tensor
    for a in range(t0, t1, chunk):
        log(f"{w.name}: filling tokens {a}..{min(t1, a + chunk)}")
        b = min(t1, a + chunk)
        k = torch.from_numpy(kv_tensor(w, 0, K, a, b)).cuda()
        v = torch.from_numpy(kv_tensor(w, 0, V, a, b)).cuda()
        tb.quantize_append(cache, k, v, a)
        if keep is not None:
            keep.append((a, k, v))
        del k, v
    torch.cuda.synchronize()


def bench_decode(tb, torch, args):
    from workloads import WORKLOADS, q_decode
    w = WORKLOADS["decode128k"]
    B, Hkv, Hq, T = w.batch, w.n_kv_heads, w.n_q_heads, w.n_ctx
    cache = tb.KVCache(B, Hkv, T)
    rows = [] if args.formats else None
    fill_cache(tb, torch, cache, w, 0, T, keep=rows)
    rng = np.random.default_rng([0, 99])
    k_new = torch.from_numpy(rng.standard_t(5, size=(B, 1, Hkv, 128)).astype(np.float32)).cuda()
    v_new = torch.from_numpy(rng.standard_t(5, size=(B, 1, Hkv, 128)).astype(np.float32)).cuda()
    q = torch.from_numpy(q_decode(w)).cuda()
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    P = args.splits or tb.decode_auto_splits(B, Hkv, T)
    ws = torch.empty(tb.decode_workspace_bytes(B, Hkv, Hq, T, P), dtype=torch.uint8, device="cuda")

    hip = HipEvents(args.steps)

    def step(i=None):
        tb.quantize_append(cache, k_new, v_new, T - 1)
        tb.attn_decode_partial(cache, q, T, w.softmax_scale, n_splits=P, workspace=ws,
                               events=None if i is None else hip.pair(i))
        tb.attn_decode_merge(ws, B, Hq, P, cache.sign_seed, out=out)

    # Under sustained load the clocks dip within ~4 ms and recover over tens
    # of ms; the settle steps run the step long enough that both timed loops
    # see the steady state rather than that transient.
    for _ in range(args.settle):
        step()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the split kernel's duration: the same steps again, with HIP events
    # recorded by every split dispatch (their markers add idle gaps around
    # the kernel, so the step time above is taken without them)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern_ms = hip.elapsed_ms()
    hip.destroy()
    # and the split kernel alone: the same K launches back to back between
    # two events on the stream they run on (no markers between launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        tb.attn_decode_partial(cache, q, T, w.softmax_scale, n_splits=P, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    kern_b2b = e0.elapsed_time(e1) / args.steps
    sweep = bench_split_sweep(tb, torch, args, cache, q, w)
    graph = bench_graph_step(tb, torch, args, cache, k_new, v_new, q, out, ws, P, w)
    verify = bench_verify(tb, torch, args, cache, w)
    formats = []
    for kf, vf in (FORMATS if args.formats else ()):
        m = tb.MixedKVCache(B, Hkv, T, kf, vf)
        for t0, k, v in rows:
            tb.mixed_append(m, k, v, t0)
        formats.append(bench_format(tb, torch, args, m, q, out, ws, P, w))
        del m
    del rows
    kv_bytes = B * T * Hkv * 2 * 66
    q_bytes = B * Hq * 128 * 4
    out_bytes = B * Hq * 128 * 2
    append_bytes = 2 * B * Hkv * 128 * 4 + 2 * B * Hkv * 66
    step_bytes = kv_bytes + q_bytes + out_bytes + append_bytes
    ms = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    achieved = (kv_bytes + q_bytes) / (kern_b2b * 1e-3) / 1e9
    assert torch.isfinite(out.float()).all()
    return {
        "P": P, "ms": ms, "value": step_bytes / (ms * 1e-3) / 1e9,
        "kernel_ms": kern_b2b, "kernel_ms_in_step": kern_avg,
        "kernel_ms_in_step_min": float(np.min(kern_ms)),
        "kernel_ms_in_step_p90": float(np.percentile(kern_ms, 90)),
        "achieved": achieved, "kv_bytes": kv_bytes, "step_bytes": step_bytes,
        "tokens_per_s": B * T / (ms * 1e-3),
        "graph": graph,
        "sweep": sweep,
        "verify": verify,
        "formats": formats,
    }


# untimed decode steps run before the warm-up steps: under sustained load the
# clocks dip within a few ms and take tens of ms to recover, so the timed steps
# start after ~0.1 s of decode (the steady state of a decode loop)
SETTLE_STEPS = 1000

# (K format, V format) pairs timed beside the TBQ4 cache on the same rows
FORMAT_NAMES = {0: "tbq4", 1: "f16", 2: "tbq3", 3: "q8_0"}
FORMATS = ((2, 2), (0, 2), (0, 1), (1, 0), (0, 3), (3, 0), (3, 3), (1, 1))
# (K format, V format) pairs of the prefill chunk timed beside TBQ4
PREFILL_FORMATS = ((2, 2), (1, 1))


def bench_format(tb, torch, args, cache, q, out, ws, P, w):
    """Decode (split kernel + merge) over a cache whose K and V tensors are
    stored in the given formats; calls back to back between two events."""
    B, T = cache.batch, cache.capacity

    def call():
        tb.mixed_attn_decode(cache, q, T, w.softmax_scale, n_splits=P, out=out, workspace=ws)

    for _ in range(args.warmup + args.settle // 10):   # clock settling, as for the step
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out.float()).all()
    kv = cache.k.numel() + cache.v.numel()
    name = f"K {FORMAT_NAMES[cache.k_format]} / V {FORMAT_NAMES[cache.v_format]}"
    log(f"decode {name}: {ms:.4f} ms/call, {kv / (ms * 1e-3) / 1e9:.0f} GB/s")
    return {"formats": name, "kv_bytes": kv, "ms_per_call": round(ms, 5),
            "kv_gbs": round(kv / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_tokens_per_s": round(B * T / (ms * 1e-3), 1)}


def bench_split_sweep(tb, torch, args, cache, q, w):
    """The split kernel alone at 98304 and 131072 attended slots of the
    resident cache, for split counts 16 .. 256 (dispatch-recorded events,
    mean over the timed calls)."""
    B, Hkv, Hq = cache.batch, cache.n_kv_heads, q.shape[1]
    res = []
    for n in (98304, cache.capacity):
        for P in (16, 32, 64, 128, 256):
            ws = torch.empty(tb.decode_workspace_bytes(B, Hkv, Hq, n, P), dtype=torch.uint8,
                             device="cuda")
            for _ in range(args.warmup):
                tb.attn_decode_partial(cache, q, n, w.softmax_scale, n_splits=P, workspace=ws)
            torch.cuda.synchronize()
            hip = HipEvents(args.steps)
            for i in range(args.steps):
                tb.attn_decode_partial(cache, q, n, w.softmax_scale, n_splits=P, workspace=ws,
                                       events=hip.pair(i))
            torch.cuda.synchronize()
            ms = float(np.mean(hip.elapsed_ms()))
            hip.destroy()
            byt = B * n * Hkv * 2 * 66 + B * Hq * 128 * 4
            res.append({"n_ctx": n, "n_splits": P, "kernel_ms": round(ms, 5),
                        "gbs": round(byt / (ms * 1e-3) / 1e9, 1)})
    log("split sweep: " + ", ".join(f"{r['n_ctx']}/{r['n_splits']}: {r['gbs']:.0f}" for r in res))
    return res


def bench_graph_step(tb, torch, args, cache, k_new, v_new, q, out, ws, P, w):
    """The same step as one captured HIP graph: append at device positions,
    then varlen decode over device lengths; replayed back to back."""
    B, T = cache.batch, cache.capacity
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")

    def step():
        tb.quantize_append_at(cache, k_new, v_new, pos)
        tb.attn_decode_varlen(cache, q, lens, T, w.softmax_scale, n_splits=P, out=out,
                              workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.settle + args.warmup):   # the same clock settling as the eager loop
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out.float()).all()
    return {"ms_per_step": ms, "replays": args.steps,
            "note": "one captured graph per step (append_at + decode_varlen), replayed back to back"}


def bench_verify(tb, torch, args, cache, w, n_q=4):
    """Multi-query verify (the current token + 3 drafted) on the same cache:
    query i attends slots [0, T - n_q + i]; one pass over the cache serves all
    n_q queries.  Reported beside n_q single-query decodes of the same bytes."""
    B, T, Hq = cache.batch, cache.capacity, w.n_q_heads
    rng = np.random.default_rng([0, 98])
    q = torch.from_numpy(rng.standard_normal((B, n_q, Hq, 128)).astype(np.float32)).cuda()
    out = torch.empty((B, n_q, Hq, 128), dtype=torch.float16, device="cuda")
    n_past = T - n_q
    ws = torch.empty(tb.verify_workspace_bytes(B, cache.n_kv_heads, Hq, n_past, n_q),
                     dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup + args.settle // 4):   # clock settling, as for the step
        tb.attn_verify(cache, q, n_past, w.softmax_scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        tb.attn_verify(cache, q, n_past, w.softmax_scale, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out.float()).all()
    kv = B * T * cache.n_kv_heads * 2 * 66
    return {"n_q": n_q, "ms_per_call": ms, "kv_gbs": kv / (ms * 1e-3) / 1e9,
            "query_tokens_per_s": B * n_q / (ms * 1e-3)}


def bench_contexts(tb, torch, args):
    """Decode steps at the two other context lengths of the workloads: 16384
    slots (batch 1, one layer; step = append one token + decode, 200 steps)
    and the long decode (batch 1, 4 layers, prefix 262080 slots, then 64
    steps that each append one token per layer and decode it over pos + 1
    slots, layers back to back).  Automatic split counts; every call goes
    through the library's decode entry point (split kernel + merge)."""
    from workloads import WORKLOADS, K, V, kv_tensor, q_decode
    res = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def kv_step_bytes(n_kv, H, Hq):
        # packed K+V attended, q in, fp16 out, the appended token (fp32 in, blocks out)
        return n_kv * H * 2 * 66 + Hq * 128 * 4 + Hq * 128 * 2 + 2 * H * (128 * 4 + 66)

    # 16K: one layer, the appended token is the workload's last row
    w = WORKLOADS["decode16k"]
    H, Hq, T = w.n_kv_heads, w.n_q_heads, w.n_ctx
    cache = tb.KVCache(1, H, T)
    k = torch.from_numpy(kv_tensor(w, 0, K, 0, T)).cuda()
    v = torch.from_numpy(kv_tensor(w, 0, V, 0, T)).cuda()
    tb.quantize_append(cache, k, v, 0)
    k_new, v_new = k[:, T - 1:].contiguous(), v[:, T - 1:].contiguous()
    q = torch.from_numpy(q_decode(w)).cuda()
    out = torch.empty((1, Hq, 128), dtype=torch.float16, device="cuda")
    ws = torch.empty(tb.decode_workspace_bytes(1, H, Hq, T, 0), dtype=torch.uint8, device="cuda")
    n = 200

    def step16():
        tb.quantize_append(cache, k_new, v_new, T - 1)
        tb.attn_decode(cache, q, T, w.softmax_scale, out=out, workspace=ws)

    for _ in range(max(args.warmup, 20)):
        step16()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        step16()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    assert torch.isfinite(out.float()).all()
    byt = kv_step_bytes(T, H, Hq)
    res.append({"workload": "decode16k: batch 1, 8 KV / 64 query heads, 16384 slots, one layer; "
                            "step = append one token + decode",
                "n_splits": tb.decode_auto_splits(1, H, T), "steps": n, "ms_per_step": round(ms, 5),
                "gbs": round(byt / (ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tokens_per_s": round(1 / (ms * 1e-3), 1)})
    log(f"decode16k: {ms:.4f} ms/step, {byt / (ms * 1e-3) / 1e9:.0f} GB/s")
    del cache, k, v, k_new, v_new, ws

    # 262K: four layers, prefix filled, then the 64 steps in the workload's order
    w = WORKLOADS["longdecode"]
    H, Hq, T0 = w.n_kv_heads, w.n_q_heads, w.n_ctx
    T = T0 + w.steps
    caches, new_k, new_v = [], [], []
    for layer in range(w.layers):
        log(f"longdecode: layer {layer}: drawing and appending {T} rows")
        c = tb.KVCache(1, H, T)
        xk = kv_tensor(w, layer, K, 0, T)
        xv = kv_tensor(w, layer, V, 0, T)
        new_k.append(torch.from_numpy(xk[:, T0:].copy()).cuda())
        new_v.append(torch.from_numpy(xv[:, T0:].copy()).cuda())
        for a in range(0, T0, 32768):
            b = min(T0, a + 32768)
            tb.quantize_append(c, torch.from_numpy(np.ascontiguousarray(xk[:, a:b])).cuda(),
                               torch.from_numpy(np.ascontiguousarray(xv[:, a:b])).cuda(), a)
        del xk, xv
        caches.append(c)
    torch.cuda.synchronize()
    qs = [[torch.from_numpy(q_decode(w, layer, st)).cuda() for st in range(w.steps)]
          for layer in range(w.layers)]
    out = torch.empty((1, Hq, 128), dtype=torch.float16, device="cuda")
    ws = torch.empty(tb.decode_workspace_bytes(1, H, Hq, T, 0), dtype=torch.uint8, device="cuda")
    for _ in range(max(args.warmup, 5)):          # warm-up on the prefix (no append)
        for layer in range(w.layers):
            tb.attn_decode(caches[layer], qs[layer][0], T0, w.softmax_scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0.record()
    for st in range(w.steps):
        pos = T0 + st
        for layer in range(w.layers):
            tb.quantize_append(caches[layer], new_k[layer][:, st:st + 1], new_v[layer][:, st:st + 1],
                               pos)
            tb.attn_decode(caches[layer], qs[layer][st], pos + 1, w.softmax_scale, out=out,
                           workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / w.steps
    assert torch.isfinite(out.float()).all()
    byt = sum(w.layers * kv_step_bytes(T0 + st + 1, H, Hq) for st in range(w.steps)) / w.steps
    res.append({"workload": "longdecode: batch 1, 8 KV / 64 query heads, 4 layers, prefix 262080 "
                            "slots, 64 steps of (append one token, decode) per layer, layers back "
                            "to back; step = all 4 layers",
                "n_splits": tb.decode_auto_splits(1, H, T), "steps": w.steps,
                "ms_per_step": round(ms, 5), "ms_per_layer": round(ms / w.layers, 5),
                "gbs": round(byt / (ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tokens_per_s": round(1 / (ms * 1e-3), 1)})
    log(f"longdecode: {ms:.4f} ms/step (4 layers), {byt / (ms * 1e-3) / 1e9:.0f} GB/s")
    del caches, new_k, new_v, qs, ws
    return res


def bench_prefill(tb, torch, args):
    from workloads import WORKLOADS, K, V, kv_tensor, q_prefill
    w = WORKLOADS["prefill"]
    n_past, n_q, Hkv, Hq = w.n_ctx, w.n_q, w.n_kv_heads, w.n_q_heads
    cache = tb.KVCache(1, Hkv, n_past + n_q)
    rows = [] if args.formats else None
    fill_cache(tb, torch, cache, w, 0, n_past, keep=rows)
    k_new = torch.from_numpy(kv_tensor(w, 0, K, n_past, n_past + n_q)).cuda()
    v_new = torch.from_numpy(kv_tensor(w, 0, V, n_past, n_past + n_q)).cuda()
    q = torch.from_numpy(q_prefill(w)).cuda()
    out = torch.empty((1, n_q, Hq, 128), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    steps = args.prefill_steps or max(3, args.steps // 4)

    def step(ev=None):
        tb.quantize_append(cache, k_new, v_new, n_past)
        if ev is not None:
            ev[0].record(stream)
        tb.attn_prefill_chunk(cache, q, n_past, w.softmax_scale, out=out)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    att_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    pairs = sum(n_past + i + 1 for i in range(n_q))
    flops = 4 * 128 * Hq * pairs
    assert torch.isfinite(out.float()).all()
    # the same chunk on caches whose K and V are TBQ3 or fp16 rows
    formats = []
    for kf, vf in (PREFILL_FORMATS if args.formats else ()):
        m = tb.MixedKVCache(1, Hkv, n_past + n_q, kf, vf)
        for t0, kc, vc in rows + [(n_past, k_new, v_new)]:
            tb.mixed_append(m, kc, vc, t0)
        for _ in range(2):
            tb.mixed_attn_prefill_chunk(m, q, n_past, w.softmax_scale, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            tb.mixed_attn_prefill_chunk(m, q, n_past, w.softmax_scale, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        assert torch.isfinite(out.float()).all()
        name = f"K {FORMAT_NAMES[kf]} / V {FORMAT_NAMES[vf]}"
        log(f"prefill {name}: {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        formats.append({"formats": name, "attention_ms": round(ms, 4),
                        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                        "frac_of_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)})
        del m
    del rows
    return {
        "workload": "prefill: 2048 new queries on 131072 cached tokens, batch 1, 8 KV / 64 Q "
                    "heads, head_dim 128; step = append of the chunk's K/V + causal attention",
        "steps": steps, "ms_per_step": wall * 1e3 / steps, "attention_ms": att_ms,
        "tflops": flops / (att_ms * 1e-3) / 1e12,
        "frac_of_mfma_peak": flops / (att_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "algorithmic_tflop": flops / 1e12, "query_tokens_per_s": n_q / (att_ms * 1e-3),
        "formats": formats,
    }


def cpu_baseline(budget_s=12.0):
    """The oracle, untuned, on whole (sequence, KV head) rows of the decode128k
    workload: fp64 dequantise of the 131072 K and V blocks + attention of the
    8 query heads.  Rate in GB/s of packed K+V consumed."""
    from oracle import tbq4_oracle as o
    from workloads import WORKLOADS, K, V, kv_rows, q_decode
    w = WORKLOADS["decode128k"]
    T, G = w.n_ctx, w.n_q_heads // w.n_kv_heads
    q = q_decode(w)
    done, spent, rows = 0, 0.0, []
    for (b, g) in [(0, 0), (1, 3), (2, 5), (3, 7), (0, 4), (1, 1)]:
        kc = o.quantize_blocks(kv_rows(w, 0, K, b, g, 0, T))[0]
        vc = o.quantize_blocks(kv_rows(w, 0, V, b, g, 0, T))[0]
        t0 = time.perf_counter()
        o.attn_decode_rows_ref(q[b, g * G:(g + 1) * G], o.dequantize_blocks(kc),
                               o.dequantize_blocks(vc), w.softmax_scale)
        spent += time.perf_counter() - t0
        done += 1
        log(f"cpu baseline: row {done} done, {spent:.1f} s")
        rows.append((b, g))
        if spent >= budget_s:
            break
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [i.get("num_threads", 1) for i in threadpool_info()])
    except Exception:
        pass
    gbs = done * T * 132 / spent / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of 32 (sequence, KV head) rows of decode128k (131072 tokens x "
                      f"8 query heads each), fp64 dequantise + attention; {spent:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on a single MI355X; sharding is a design note only)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_attention_tbq4_amd as tb
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}))
        return
    dec = bench_decode(tb, torch, args)
    log(f"decode: {dec['ms']:.4f} ms/step, kernel {dec['kernel_ms']:.4f} ms, "
        f"{dec['achieved']:.0f} GB/s")
    ctx = None if args.no_contexts else bench_contexts(tb, torch, args)
    pre = None if args.no_prefill else bench_prefill(tb, torch, args)
    if pre:
        log(f"prefill: {pre['attention_ms']:.3f} ms, {pre['tflops']:.1f} TFLOP/s")
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode128k: batch 4 sequences, 8 KV / 64 query heads, head_dim 128, "
                        "131072 cached tokens in TBQ4 K and V (Student-t nu=5 x per-channel "
                        "scales); step = append one token per sequence + split-K decode",
            "batch": 4, "n_ctx": 131072, "n_kv_heads": 8, "n_q_heads": 64, "n_splits": dec["P"],
            "hbm_frac_of_step": round(dec["value"] / HBM_PEAK_GBS, 4),
            "kv_tokens_per_s": round(dec["tokens_per_s"], 1),
        },
        "verify": {
            "workload": "decode128k cache, 4 queries per sequence (1 + 3 drafted), query i "
                        "attends slots [0, 131068 + i]; calls back to back (launch + merge)",
            "ms_per_call": round(dec["verify"]["ms_per_call"], 5),
            "kv_gbs": round(dec["verify"]["kv_gbs"], 1),
            "query_tokens_per_s": round(dec["verify"]["query_tokens_per_s"], 1),
            "vs_4_decodes": round(4 * dec["ms"] / dec["verify"]["ms_per_call"], 3),
        },
        "formats": {
            "workload": "decode128k rows stored per tensor as TBQ4 (66 B), TBQ3 (50 B), "
                        "q8_0 (136 B) or fp16 (256 B) per head vector; one decode call (split "
                        "kernel + merge) over 131072 slots, calls back to back",
            "results": dec["formats"],
        },
        "split_sweep": {
            "workload": "decode128k cache; split kernel alone at 98304 and 131072 attended "
                        "slots, batch 4, 8 / 64 heads",
            "results": dec["sweep"],
        },
        "graph_step": {
            "ms_per_step": round(dec["graph"]["ms_per_step"], 5),
            "value": round(dec["step_bytes"] / (dec["graph"]["ms_per_step"] * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "note": dec["graph"]["note"],
        },
        "roofline": {
            "kernel": "decode_split_kernel",
            "bound": "hbm",
            "achieved": round(dec["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dec["P"]),
            "kernel_ms": round(dec["kernel_ms"], 5),
            "kernel_ms_in_step": round(dec["kernel_ms_in_step"], 5),
            "kernel_ms_in_step_min": round(dec["kernel_ms_in_step_min"], 5),
            "kernel_ms_in_step_p90": round(dec["kernel_ms_in_step_p90"], 5),
            "timing": "kernel_ms: K launches of the split kernel back to back between two "
                      "HIP events on the stream they run on, right after the timed steps; "
                      "kernel_ms_in_step: HIP events recorded by the split kernel's own "
                      "dispatch (hipExtLaunchKernel) on every step of a second loop of the "
                      "same K steps (their markers add a few microseconds per call)",
        },
        "cpu_baseline": cpu,
        "contexts": ctx,
        "prefill": pre,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
