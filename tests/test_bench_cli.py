"""bench.py's host-side contract, on the CPU: more than one GPU is refused with
a message, and the CPU baseline (the oracle timed on a bounded sample of the
128K decode workload) reports the fields the result line carries."""

import importlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    # imported by name, so that worker processes of the CPU legs can import
    # the functions they run
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    return importlib.import_module("bench")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                        "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    bench = _bench_module()
    cpu = bench.cpu_baseline(quick=True)   # one row per leg
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s"
    assert cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["host_cpus"] >= 1
    assert cpu["sample"].startswith("1 of the 32 (sequence, KV head) rows of one decode128k call")
    legs = cpu["legs"]
    for k in ("quantize", "tiny", "decode16k", "decode_98304", "decode_131072", "longdecode_step",
              "prefill"):
        assert k in legs, k
    assert legs["quantize"]["blocks_per_s_1_thread"] > 0
    assert legs["prefill"]["s_per_chunk_extrapolated"] > 0


def test_traffic_only_for_the_measured_split_count():
    bench = _bench_module()
    assert bench.measured_traffic(bench.TRAFFIC["n_splits"] + 1) is None
    t = bench.measured_traffic(bench.TRAFFIC["n_splits"])
    # either the sources are the measured ones (bytes per launch at least the
    # algorithmic 553 779 200 B) or they changed since (unknown: None)
    assert t is None or t >= 553_779_200


def test_defaults_settle_and_switches(monkeypatch):
    bench = _bench_module()
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.splits) == (1, 200, 20, 0)
    assert a.settle == bench.SETTLE_STEPS >= 600   # timed steps start after the clock dip
    monkeypatch.setattr(sys, "argv", ["bench.py", "--settle", "60", "--no-contexts", "--no-prefill"])
    a = bench.parse()
    assert a.settle == 60 and a.no_contexts and a.no_prefill
