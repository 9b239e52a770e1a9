"""Benchmark of the TBQ4 attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--splits P] [--settle S]
                    [--no-prefill] [--no-cpu-baseline] [--no-formats] [--no-contexts]

One step = one pass of the whole decode hot path over the decode128k workload
(batch 4 independent sequences, 8 KV / 64 query heads, head_dim 128, 131072
cached tokens in TBQ4 K and V caches resident in HBM): quantise-append the new
token's K and V for every sequence and split-K decode attention over all
131072 slots, as one tbq4_decode_step call (the split kernel, whose extra
wavefronts quantise, store and score the new token, then the merge kernel).
The headline value is the step's algorithmic HBM bytes (packed K+V read, q
read, output written, appended rows) divided by the step time, in GB/s; the
same step as three launches (append, split kernel, merge) is timed beside it.
The prefill-chunk workload (2048 queries on 131072 cached tokens, 8 KV / 64
query heads, append of the chunk's K/V then causal attention) is timed in the
same run and reported under "prefill" in TFLOP/s (4 * 128 * 64 FLOPs per
unmasked (query, key) pair).  The same decode rows stored as TBQ3, q8_0 or
fp16 K / V tensors (mixed formats) are timed under "formats" (one decode call
per format pair, KV GB/s), and the prefill chunk over TBQ3 and fp16 caches
under "prefill"."formats".  Decode at 16384 slots (batch 1) and the 4-layer
long decode at 262144 slots (batch 1, 64 decode steps per layer) are timed
under "contexts".

Before the W warm-up steps, S untimed steps (default 1000, ~0.12 s) let the
clocks settle: the first milliseconds of sustained load run faster, then the
clocks dip and recover over tens of milliseconds.  The step value is timed
over K steps (default 200, ~23 ms) without any event markers.  A second loop
of the same K steps records HIP events from the dispatch of every split
kernel (start and end of that kernel's execution): their mean is the
roofline's kernel_ms, and the kernel's algorithmic bytes over it the
roofline's achieved rate.  The plain split kernel is also timed inside K
three-launch steps and K times back to back with no gaps.
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

# HBM bytes per launch of the decode step's split kernel on this workload (64
# streaming splits + the new-token wavefronts), from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) scaled by what the same
# counters read for a plain 256 MiB device copy (FETCH_SIZE reads half the
# copied bytes -> x2.0; WRITE_SIZE reads them all -> x1.0).  Reported only while
# the kernel's sources hash to the version the counters were taken on;
# otherwise the traffic is unknown (null).
KERNEL_SOURCES = ("decode.hip", "tbq4_device.h", "tbq4_launch.h")
TRAFFIC = {"sources_sha256": "a21e7c620ca1b13449fd852ef52e8acc2bbbc5ec6ec644a34074ab3851a0e758",
           "n_splits": 64, "fetch_kib": 271259.7, "fetch_factor": 2.0,
           "write_kib": 8852.3, "write_factor": 1.0}


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
    # 200 timed steps (~23 ms): a window long enough that a clock transient of
    # a few ms does not decide the step time
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
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
    p.add_argument("--prefill-only", action="store_true",
                   help="only time the prefill chunk (for profiler passes over that kernel) and "
                        "print its measurements as one JSON line")
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


def dist(ms):
    """median, p10 and p90 of a list of per-call times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


class Flush:
    """Reads a 1 GiB buffer (untimed, on the same stream, before the first
    event of a timed call) with the library's streaming-read helper, which
    evicts the 256 MB Infinity Cache and the L2s with clean lines: the call
    that follows reads its inputs from HBM.  (Writing the buffer instead
    leaves ~256 MB of dirty lines whose write-back then competes with the
    timed call's reads.)"""

    def __init__(self, torch):
        import ctypes
        import long_context_attention_tbq4_amd as tb
        self.ct = ctypes
        self.L = tb._lib.lib()
        self.torch = torch
        self.buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        self.sink = torch.empty(512, dtype=torch.int32, device="cuda")

    def __call__(self):
        st = self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        rc = self.L.tbq4_bench_stream_read(self.ct.c_void_p(self.buf.data_ptr()), self.buf.numel(),
                                           self.ct.c_void_p(self.sink.data_ptr()), 512, st)
        assert rc == 0, rc


def time_each(torch, fn, n, flush=None):
    """Per-call times (ms) of n calls of fn, each between two events on the
    current stream; with `flush`, the flush runs before each call's first
    event (outside the timed interval)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def manifest_clocks():
    """Current core, memory and fabric clock levels from the driver's sysfs
    tables (the level marked '*'), per GPU card; None where unreadable."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        card = {}
        for clk in ("sclk", "mclk", "fclk", "socclk"):
            try:
                with open(os.path.join(dev, "pp_dpm_" + clk)) as f:
                    cur = [l.split(":", 1)[1].strip(" *\n") for l in f if l.rstrip().endswith("*")]
                card[clk] = cur[0] if cur else None
            except (OSError, IndexError):
                pass
        if card:
            out[os.path.basename(os.path.dirname(dev))] = card
    return out or None


def git_head(root):
    """Commit of the working tree, read from .git without running git."""
    try:
        with open(os.path.join(root, ".git", "HEAD")) as f:
            ref = f.read().strip()
        if not ref.startswith("ref: "):
            return ref or None
        name = ref[5:]
        path = os.path.join(root, ".git", name)
        if os.path.exists(path):
            with open(path) as f:
                return f.read().strip() or None
        with open(os.path.join(root, ".git", "packed-refs")) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 2 and parts[1] == name:
                    return parts[0]
    except OSError:
        pass
    return None


def manifest(torch):
    """What the numbers were measured on: ROCm, device, clocks, sources."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    m = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            m["rocm"] = f.read().strip()
    except OSError:
        m["rocm"] = None
    props = torch.cuda.get_device_properties(0)
    m["device"] = props.name
    m["gfx_arch"] = getattr(props, "gcnArchName", None)
    m["compute_units"] = props.multi_processor_count
    m["hbm_bytes"] = props.total_memory
    m["clocks_idle"] = manifest_clocks()
    h = hashlib.sha256()
    for sub in ("long_context_attention_tbq4_amd/csrc", "include"):
        d = os.path.join(root, sub)
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    m["sources_sha256"] = h.hexdigest()
    m["git_head"] = git_head(root)   # None where the tree was copied without .git
    m["host_cpus"] = len(os.sched_getaffinity(0))
    return m


def bench_denominators(tb, torch):
    """Measured-achievable peaks: a read-only streaming kernel over 1 GiB
    (best of four grid sizes) and an MFMA-only loop of independent fp16
    32x32x16 products (best of three grid sizes)."""
    import ctypes
    L = tb._lib.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = 1 << 30
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1 << 18, dtype=torch.float32, device="cuda")
    read = []
    for nb in (256, 512, 1024, 2048):
        def rd():
            assert L.tbq4_bench_stream_read(ctypes.c_void_p(buf.data_ptr()), n,
                                            ctypes.c_void_p(sink.data_ptr()), nb, st) == 0
        for _ in range(3):
            rd()
        ms = float(np.median(time_each(torch, rd, 10)))
        read.append({"workgroups": nb, "ms": round(ms, 5), "gbs": round(n / (ms * 1e-3) / 1e9, 1)})
    mf = []
    iters = 2000
    for nb in (256, 512, 1024):
        def mm():
            assert L.tbq4_bench_mfma_f16(iters, ctypes.c_void_p(sink.data_ptr()), nb, st) == 0
        for _ in range(2):
            mm()
        ms = float(np.median(time_each(torch, mm, 5)))
        flops = nb * 4 * iters * 8 * 32768
        mf.append({"workgroups": nb, "ms": round(ms, 5),
                   "tflops": round(flops / (ms * 1e-3) / 1e12, 1)})
    del buf, sink
    best_r = max(read, key=lambda r: r["gbs"])
    best_m = max(mf, key=lambda r: r["tflops"])
    log(f"achievable: stream read {best_r['gbs']:.0f} GB/s, fp16 MFMA {best_m['tflops']:.0f} TFLOP/s")
    return {"stream_read_gbs": best_r["gbs"], "mfma_f16_tflops": best_m["tflops"],
            "stream_read": read, "mfma_f16": mf,
            "note": "stream: 1 GiB read once, 16-byte non-temporal loads, 4 in flight per lane; "
                    "mfma: 8 independent v_mfma_f32_32x32x16_f16 chains per wavefront, "
                    "register operands; medians of back-to-back calls"}


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
    ws = torch.empty(tb.decode_step_workspace_bytes(B, Hkv, Hq, T, P), dtype=torch.uint8,
                     device="cuda")

    hip = HipEvents(args.steps)

    hip3 = HipEvents(args.steps)

    def step(i=None):
        """the decode step: the new token appended and attended in the split
        kernel's launch (two extra wavefronts per (sequence, KV head)), then
        the merge; with i, the split kernel's dispatch records HIP events"""
        tb.decode_step(cache, k_new, v_new, q, T - 1, w.softmax_scale, n_splits=P, out=out,
                       workspace=ws, events=None if i is None else hip.pair(i))

    def step_unfused(i=None):
        """the same step as three launches: append, split kernel, merge"""
        tb.quantize_append(cache, k_new, v_new, T - 1)
        tb.attn_decode_partial(cache, q, T, w.softmax_scale, n_splits=P, workspace=ws,
                               events=None if i is None else hip3.pair(i))
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
    # the step's split kernel inside the steps: the same K steps again, each
    # split dispatch recording HIP events (their markers add small idle gaps
    # around the kernel, so the step time above is taken without them)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern_ms = hip.elapsed_ms()
    hip.destroy()
    # the same steps as three launches (append, split kernel, merge), and the
    # plain split kernel's duration inside them
    for _ in range(args.warmup):
        step_unfused()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_unfused()
    torch.cuda.synchronize()
    wall_unfused = time.perf_counter() - t0
    for i in range(args.steps):
        step_unfused(i)
    torch.cuda.synchronize()
    kern3_ms = hip3.elapsed_ms()
    hip3.destroy()
    # and the plain split kernel alone: K launches back to back between two
    # events on the stream they run on (no markers, no gaps: the hottest
    # case for the clocks)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        tb.attn_decode_partial(cache, q, T, w.softmax_scale, n_splits=P, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    kern_b2b = e0.elapsed_time(e1) / args.steps
    # per-step and per-kernel distributions: warm (back to back, the cache
    # partly resident in the Infinity Cache) and cold (1 GiB read before
    # every timed call)
    flush = Flush(torch)
    split = lambda: tb.attn_decode_partial(cache, q, T, w.softmax_scale, n_splits=P, workspace=ws)
    n_d = max(args.steps, 50)
    dists = {"step_warm": dist(time_each(torch, step, n_d)),
             "step_cold": dist(time_each(torch, step, n_d, flush)),
             "split_kernel_warm": dist(time_each(torch, split, n_d)),
             "split_kernel_cold": dist(time_each(torch, split, n_d, flush))}
    del flush
    log("decode128k per-call ms: " + ", ".join(f"{k} {v['median']:.4f}" for k, v in dists.items()))
    share = bench_share(tb, torch, args, cache, q, w)
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
    ms_unfused = wall_unfused * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    # the step's split kernel: packed K+V of the T - 1 slots before the new
    # token, the queries, the new token's fp32 K and V rows and its two blocks
    kernel_bytes = (B * (T - 1) * Hkv * 2 * 66 + q_bytes + 2 * B * Hkv * 128 * 4
                    + 2 * B * Hkv * 66)
    achieved = kernel_bytes / (kern_avg * 1e-3) / 1e9
    assert torch.isfinite(out.float()).all()
    return {
        "P": P, "ms": ms, "value": step_bytes / (ms * 1e-3) / 1e9, "ms_unfused": ms_unfused,
        "kernel_ms": kern_avg, "kernel_ms_min": float(np.min(kern_ms)),
        "kernel_ms_p90": float(np.percentile(kern_ms, 90)),
        "kernel_ms_three_launch_step": float(np.mean(kern3_ms)),
        "kernel_ms_b2b_plain": kern_b2b, "kernel_bytes": kernel_bytes,
        "achieved": achieved, "kv_bytes": kv_bytes, "step_bytes": step_bytes,
        "tokens_per_s": B * T / (ms * 1e-3),
        "graph": graph,
        "dists": dists,
        "share": share,
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


def bench_share(tb, torch, args, cache, q, w):
    """One GPU's share when the decode128k heads are sharded over 8 GPUs:
    batch 4, 1 KV head / 8 query heads, 131072 slots (KV head 0 of the
    resident cache, copied untimed), split kernel + merge at 128 and 256
    splits and the automatic count; calls back to back."""
    B, T = cache.batch, cache.capacity
    c1 = tb.KVCache(B, 1, T)
    c1.k.copy_(cache.k[:, 0:1])
    c1.v.copy_(cache.v[:, 0:1])
    q1 = q[:, 0:8].contiguous()
    out = torch.empty((B, 8, 128), dtype=torch.float16, device="cuda")
    kv = B * T * 2 * 66
    res = []
    for P in (128, 256, 0):
        Pu = P or tb.decode_auto_splits(B, 1, T)
        ws = torch.empty(tb.decode_workspace_bytes(B, 1, 8, T, Pu), dtype=torch.uint8, device="cuda")
        call = lambda: tb.attn_decode(c1, q1, T, w.softmax_scale, n_splits=Pu, out=out, workspace=ws)
        part = lambda: tb.attn_decode_partial(c1, q1, T, w.softmax_scale, n_splits=Pu, workspace=ws)
        for _ in range(args.warmup + args.settle // 10):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        e0.record()
        for _ in range(args.steps):
            part()
        e1.record()
        torch.cuda.synchronize()
        kms = e0.elapsed_time(e1) / args.steps
        res.append({"n_splits": Pu, "ms_per_call": round(ms, 5), "kernel_ms": round(kms, 5),
                    "gbs": round(kv / (ms * 1e-3) / 1e9, 1),
                    "kernel_gbs": round((kv + B * 8 * 512) / (kms * 1e-3) / 1e9, 1),
                    "kernel_frac_of_hbm_peak": round((kv + B * 8 * 512) / (kms * 1e-3) / 1e9
                                                     / HBM_PEAK_GBS, 4)})
    assert torch.isfinite(out.float()).all()
    del c1, q1
    log("share (1 KV head / 8 q heads): " + ", ".join(f"P={r['n_splits']}: {r['gbs']:.0f}" for r in res))
    return {"workload": "one GPU's share of decode128k sharded by KV head over 8 GPUs: batch 4, "
                        "1 KV / 8 query heads, 131072 slots; decode call (split kernel + merge) "
                        "back to back, and the split kernel alone",
            "kv_bytes": kv, "results": res}


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
    """The same step as one captured HIP graph, the new token's slot read
    from device memory; replayed back to back."""
    B, T = cache.batch, cache.capacity
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")

    def step():
        tb.decode_step(cache, k_new, v_new, q, T - 1, w.softmax_scale, positions=pos,
                       n_splits=P, out=out, workspace=ws)

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
            "note": "one captured graph per step (the decode step at device positions: split "
                    "kernel with the new-token wavefronts + merge), replayed back to back"}


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
    slots, layers back to back).  Automatic split counts; every step goes
    through the library's decode-step entry point (the split kernel with the
    new-token wavefronts, then the merge)."""
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
    ws = torch.empty(tb.decode_step_workspace_bytes(1, H, Hq, T, 0), dtype=torch.uint8,
                     device="cuda")
    n = 200

    def step16():
        tb.decode_step(cache, k_new, v_new, q, T - 1, w.softmax_scale, out=out, workspace=ws)

    for _ in range(max(args.warmup, 20) + args.settle):   # clock settling, as for decode128k
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
    # the 17 MB cache fits in the 256 MB Infinity Cache: cold steps read
    # 1 GiB before each timed step
    flush = Flush(torch)
    d16 = {"step_warm": dist(time_each(torch, step16, 100)),
           "step_cold": dist(time_each(torch, step16, 100, flush))}
    del flush
    log(f"decode16k per-step ms: warm {d16['step_warm']['median']:.4f}, "
        f"cold {d16['step_cold']['median']:.4f}")
    res.append({"workload": "decode16k: batch 1, 8 KV / 64 query heads, 16384 slots, one layer; "
                            "step = append one token + decode",
                "per_step_ms": d16,
                "cold_gbs": round(byt / (d16["step_cold"]["median"] * 1e-3) / 1e9, 1),
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
    ws = torch.empty(tb.decode_step_workspace_bytes(1, H, Hq, T, 0), dtype=torch.uint8,
                     device="cuda")
    for _ in range(max(args.warmup, 5)):          # warm-up on the prefix (no append)
        for layer in range(w.layers):
            tb.attn_decode(caches[layer], qs[layer][0], T0, w.softmax_scale, out=out, workspace=ws)

    def run_steps():
        for st in range(w.steps):
            pos = T0 + st
            for layer in range(w.layers):
                tb.decode_step(caches[layer], new_k[layer][:, st:st + 1],
                               new_v[layer][:, st:st + 1], qs[layer][st], pos, w.softmax_scale,
                               out=out, workspace=ws)

    # clock settling, as for decode128k: the 64-step sequence itself, run
    # untimed (each step writes its token's slot and attends only up to it, so
    # a repeat computes and writes exactly what the first pass did)
    for _ in range(max(1, args.settle // 250)):
        run_steps()
    torch.cuda.synchronize()
    e0.record()
    run_steps()
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
    steps = args.prefill_steps or 20   # timed calls, warm and cold alike

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
    att_list = [a.elapsed_time(b) for a, b in evs]
    att_ms = float(np.mean(att_list))
    pairs = sum(n_past + i + 1 for i in range(n_q))
    flops = 4 * 128 * Hq * pairs
    assert torch.isfinite(out.float()).all()
    # cold attention calls (1 GiB read before each; the 141 MB cache would
    # otherwise sit in the Infinity Cache) and the chunk's quantise-append
    flush = Flush(torch)
    att_cold = time_each(torch, lambda: tb.attn_prefill_chunk(cache, q, n_past, w.softmax_scale,
                                                              out=out), steps, flush)
    app = lambda: tb.quantize_append(cache, k_new, v_new, n_past)
    app_warm = time_each(torch, app, 20)
    app_cold = time_each(torch, app, 20, flush)
    del flush
    app_bytes = 2 * n_q * Hkv * 128 * 4 + 2 * n_q * Hkv * 66     # fp32 rows in, blocks out
    app_blocks = 2 * n_q * Hkv
    log(f"prefill attention cold {np.median(att_cold):.3f} ms; append {np.median(app_warm):.4f} ms")
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
        "attention_ms_warm": dist(att_list), "attention_ms_cold": dist(att_cold),
        "tflops_cold": flops / (float(np.median(att_cold)) * 1e-3) / 1e12,
        "append": {"workload": "quantise-append of the chunk: 2048 tokens x 8 KV heads, K and V "
                               "(fp32 rows in, 66-byte blocks out)",
                   "blocks": app_blocks, "bytes": app_bytes,
                   "ms_warm": dist(app_warm), "ms_cold": dist(app_cold),
                   "gbs_warm": round(app_bytes / (float(np.median(app_warm)) * 1e-3) / 1e9, 1),
                   "gbs_cold": round(app_bytes / (float(np.median(app_cold)) * 1e-3) / 1e9, 1),
                   "blocks_per_s": round(app_blocks / (float(np.median(app_warm)) * 1e-3), 1)},
        "tflops": flops / (att_ms * 1e-3) / 1e12,
        "frac_of_mfma_peak": flops / (att_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "algorithmic_tflop": flops / 1e12, "query_tokens_per_s": n_q / (att_ms * 1e-3),
        "formats": formats,
    }


# --------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on the host's cores.  Each leg
# times one oracle call (dequantise the packed rows + softmax attention) on
# inputs prepared beforehand (generated and quantised, untimed); rows are
# spread over worker processes (one BLAS thread each), so `cores` is the
# number of workers.
# --------------------------------------------------------------------------
def _cpu_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([1] + [i.get("num_threads", 1) for i in threadpool_info()])
    except Exception:
        return None


def _cpu_quantize_job(n_blocks):
    """fp64 quantiser on n seeded N(0,1) blocks: (blocks, seconds).  (numpy
    element-wise work: one thread per process.)"""
    from oracle import tbq4_oracle as o
    x = np.random.default_rng([0, 77, n_blocks]).standard_normal((n_blocks, 128)).astype(np.float32)
    t0 = time.perf_counter()
    o.quantize_blocks(x)
    return n_blocks, time.perf_counter() - t0


def _cpu_row_prep(args):
    """Generate and quantise one (layer, sequence, KV head) row of a decode
    workload (untimed preparation): returns the packed K, V rows."""
    _one_blas_thread()
    from oracle import tbq4_oracle as o
    from workloads import WORKLOADS, K, V, kv_rows
    wname, layer, b, g, t_end = args
    w = WORKLOADS[wname]
    return (o.quantize_blocks(kv_rows(w, layer, K, b, g, 0, t_end))[0],
            o.quantize_blocks(kv_rows(w, layer, V, b, g, 0, t_end))[0])


def _cpu_row_call(args):
    """The timed oracle work of one row: dequantise the packed rows and run
    softmax attention for each (q_rows, n) asked for.  Returns seconds."""
    _one_blas_thread()
    from oracle import tbq4_oracle as o
    kc, vc, jobs, scale = args
    t0 = time.perf_counter()
    Kd, Vd = o.dequantize_blocks(kc), o.dequantize_blocks(vc)
    for qr, n in jobs:
        o.attn_decode_rows_ref(qr, Kd[:n], Vd[:n], scale)
    return time.perf_counter() - t0


def cpu_baseline(quick=False):
    """The oracle's legs; `quick` (for the host-side test) shrinks every
    sample to a row or a few blocks."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from oracle import tbq4_oracle as o
    from workloads import WORKLOADS, K, V, kv_rows, kv_tensor, q_decode, q_prefill, tiny_inputs
    nw = _cpu_workers()
    legs = {}
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(nw, mp_context=ctx) as ex:
        # quantise: one process, then all workers at once
        nq = 512 if quick else 32768
        n1, s1 = _cpu_quantize_job(nq)
        t0 = time.perf_counter()
        done = sum(n for n, _ in ex.map(_cpu_quantize_job, [nq] * nw))
        wall = time.perf_counter() - t0
        legs["quantize"] = {"blocks_per_s_1_thread": round(n1 / s1, 1),
                            "blocks_per_s_all": round(done / wall, 1), "workers": nw,
                            "sample": f"{nq} seeded N(0,1) blocks per process"}
        log(f"cpu baseline: quantize {n1 / s1:.0f} blocks/s (1 thread), {done / wall:.0f} ({nw})")

        def prepare(wname, layer_heads, t_end):
            return list(ex.map(_cpu_row_prep, [(wname, l, b, g, t_end) for l, b, g in layer_heads]))

        def decode_call(wname, layer_heads, n, qfn, prep):
            """the (layer, b, g) rows of one call, prepared beforehand: time
            the call with the rows spread over the workers"""
            w = WORKLOADS[wname]
            G = w.n_q_heads // w.n_kv_heads
            jobs = [(kc, vc, [(qfn(l)[b, g * G:(g + 1) * G], n)], w.softmax_scale)
                    for (l, b, g), (kc, vc) in zip(layer_heads, prep)]
            t0 = time.perf_counter()
            cpu_s = sum(ex.map(_cpu_row_call, jobs))
            return time.perf_counter() - t0, cpu_s

        # C1: the tiny workload, whole (one process)
        k, v, q, _ = tiny_inputs()
        kc = o.quantize_blocks(k.transpose(0, 2, 1, 3))[0]
        vc = o.quantize_blocks(v.transpose(0, 2, 1, 3))[0]
        t0 = time.perf_counter()
        o.attn_decode_ref(q, kc, vc, 1024, WORKLOADS["tiny"].softmax_scale)
        legs["tiny"] = {"ms_per_call": round((time.perf_counter() - t0) * 1e3, 3), "workers": 1}
        # C2: decode16k, one whole call (8 KV heads)
        w = WORKLOADS["decode16k"]
        rows = [(0, 0, g) for g in range(1 if quick else 8)]
        wall, cs = decode_call("decode16k", rows, w.n_ctx, lambda l: q_decode(w),
                               prepare("decode16k", rows, w.n_ctx))
        legs["decode16k"] = {"s_per_call": round(wall, 3), "cpu_s": round(cs, 3), "workers": nw,
                             "rows": len(rows), "gbs": round(w.n_ctx * len(rows) * 132 / wall / 1e9, 4)}
        log(f"cpu baseline: decode16k {wall:.2f} s per call")
        # C3: one call at 98304 and at 131072 slots (all 32 rows)
        w = WORKLOADS["decode128k"]
        rows = [(0, b, g) for b in range(1 if quick else 4) for g in range(1 if quick else 8)]
        prep = prepare("decode128k", rows, 131072)    # the 98304-slot call reads a prefix
        for n in (98304, 131072):
            wall, cs = decode_call("decode128k", rows, n, lambda l: q_decode(w), prep)
            legs[f"decode_{n}"] = {"s_per_call": round(wall, 3), "cpu_s": round(cs, 3),
                                   "workers": nw, "rows": len(rows),
                                   "gbs": round(len(rows) * n * 132 / wall / 1e9, 4)}
            log(f"cpu baseline: decode {n} {wall:.2f} s per call")
        del prep
        # C5: one long-decode step at its first position: layer 0 measured
        # (8 KV heads), the 4-layer step is that x 4
        w = WORKLOADS["longdecode"]
        n5 = w.n_ctx + 1
        rows = [(0, 0, g) for g in range(1 if quick else 8)]
        wall, cs = decode_call("longdecode", rows, n5, lambda l: q_decode(w, l, 0),
                               prepare("longdecode", rows, n5))
        legs["longdecode_step"] = {"s_one_layer": round(wall, 3), "s_per_step_x4": round(4 * wall, 3),
                                   "cpu_s": round(cs, 3), "workers": nw,
                                   "rows": len(rows), "gbs": round(n5 * len(rows) * 132 / wall / 1e9, 4),
                                   "note": "layer 0 of step 0 (8 KV heads at 262081 slots) measured; "
                                           "the 4-layer step is that x 4 (extrapolated)"}
        log(f"cpu baseline: long-decode layer {wall:.2f} s")
    # C4: one KV-head group of the prefill chunk (all 2048 queries), x 8;
    # numpy's BLAS on nw threads in this process
    w = WORKLOADS["prefill"]
    T = w.n_ctx + w.n_q
    kc = o.quantize_blocks(kv_rows(w, 0, K, 0, 0, 0, T))[0]
    vc = o.quantize_blocks(kv_rows(w, 0, V, 0, 0, 0, T))[0]
    stride = 512 if quick else 16
    rows = np.arange(0, w.n_q, stride)              # 128 of the 2048 chunk rows
    qg = q_prefill(w)[0][rows, 0:8]
    from threadpoolctl import threadpool_limits
    with threadpool_limits(nw):
        t0 = time.perf_counter()
        Kd, Vd = o.dequantize_blocks(kc), o.dequantize_blocks(vc)
        o.attn_prefill_rows_ref(qg, Kd, Vd, w.n_ctx, rows, w.softmax_scale)
        grp = time.perf_counter() - t0
    flops = 4 * 128 * 64 * sum(w.n_ctx + i + 1 for i in range(w.n_q))
    est = grp * stride * 8
    legs["prefill"] = {"s_sample": round(grp, 3), "s_per_chunk_extrapolated": round(est, 1),
                       "tflops": round(flops / est / 1e12, 6), "blas_threads": nw,
                       "note": "KV-head group 0, every 16th of the 2048 chunk queries (128 rows x 8 "
                               "heads, dequantise + causal attention) measured; the chunk is that "
                               "x 16 x 8 (extrapolated)"}
    log(f"cpu baseline: prefill sample {grp:.2f} s (chunk ~{est:.0f} s)")
    del Kd, Vd
    head = legs["decode_131072"]
    return {"value": head["gbs"], "unit": "GB/s", "cores": nw, "kind": "oracle",
            "sample": f"{head['rows']} of the 32 (sequence, KV head) rows of one decode128k call "
                      "at 131072 slots (packed K+V, 8 query heads each): fp64 dequantise + softmax "
                      f"attention, rows spread over {nw} worker processes with one BLAS thread "
                      f"each; {head['s_per_call']} s",
            "host_cpus": len(os.sched_getaffinity(0)), "blas_threads_default": _blas_threads(),
            "legs": legs}


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
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(tb, torch, args)}), flush=True)
        return
    man = manifest(torch)
    den = bench_denominators(tb, torch)
    dec = bench_decode(tb, torch, args)
    man["clocks_after_decode"] = manifest_clocks()
    log(f"decode: {dec['ms']:.4f} ms/step, kernel {dec['kernel_ms']:.4f} ms, "
        f"{dec['achieved']:.0f} GB/s")
    ctx = None if args.no_contexts else bench_contexts(tb, torch, args)
    pre = None if args.no_prefill else bench_prefill(tb, torch, args)
    if pre:
        log(f"prefill: {pre['attention_ms']:.3f} ms, {pre['tflops']:.1f} TFLOP/s")
        pre["frac_of_achievable_mfma"] = pre["tflops"] / den["mfma_f16_tflops"]
        pre["achievable_mfma_tflops"] = den["mfma_f16_tflops"]
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "ms_per_step_three_launches": round(dec["ms_unfused"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode128k: batch 4 sequences, 8 KV / 64 query heads, head_dim 128, "
                        "131072 cached tokens in TBQ4 K and V (Student-t nu=5 x per-channel "
                        "scales); step = append one token per sequence + split-K decode, as "
                        "one decode-step call (split kernel whose extra wavefronts quantise, store "
                        "and score the new token, then the merge)",
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
        "per_call_ms": {
            "workload": "decode128k; step = one decode-step call (split kernel with the new-token "
                        "wavefronts + merge); warm: back to back "
                        "(part of the cache stays in the 256 MB Infinity Cache), cold: 1 GiB "
                        "read before each timed call; each call between two HIP events",
            **dec["dists"],
            "step_cold_gbs": round(dec["step_bytes"] / (dec["dists"]["step_cold"]["median"] * 1e-3)
                                   / 1e9, 1),
            "split_kernel_cold_gbs": round((dec["kv_bytes"] + 4 * 64 * 512)
                                           / (dec["dists"]["split_kernel_cold"]["median"] * 1e-3)
                                           / 1e9, 1),
        },
        "share_1_of_8_gpus": dec["share"],
        "achievable": den,
        "manifest": man,
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
            "kernel": "decode_split_kernel (the decode step's launch: 64 streaming splits and "
                      "the new-token wavefronts)",
            "bound": "hbm",
            "achieved": round(dec["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec["achieved"] / HBM_PEAK_GBS, 4),
            "frac_of_achievable": round(dec["achieved"] / den["stream_read_gbs"], 4),
            "achievable_peak": den["stream_read_gbs"],
            "traffic": measured_traffic(dec["P"]),
            "kernel_bytes": dec["kernel_bytes"],
            "kernel_ms": round(dec["kernel_ms"], 5),
            "kernel_ms_min": round(dec["kernel_ms_min"], 5),
            "kernel_ms_p90": round(dec["kernel_ms_p90"], 5),
            "kernel_ms_three_launch_step": round(dec["kernel_ms_three_launch_step"], 5),
            "kernel_ms_b2b_plain": round(dec["kernel_ms_b2b_plain"], 5),
            "timing": "kernel_ms: mean of the HIP events that the split kernel's own dispatch "
                      "(hipExtLaunchKernel) records in each of K decode steps run right after "
                      "the timed ones; achieved = kernel_bytes / kernel_ms. "
                      "kernel_ms_three_launch_step: the same for the plain split kernel inside "
                      "K three-launch steps; kernel_ms_b2b_plain: K plain split kernels back to "
                      "back between two events, no gaps (the hottest case for the clocks)",
        },
        "cpu_baseline": cpu,
        "contexts": ctx,
        "prefill": pre,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
