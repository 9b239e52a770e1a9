"""The C ABI end to end on the GPU: tests/c/abi_gpu_decode.c (plain C, gcc,
the HIP runtime's C API for device memory) quantise-appends seeded K/V rows and
runs decode attention, and the one-call decode step, through include/tbq4.h;
its packed caches must be the oracle's bytes and its outputs must meet the
attention bar against the fp64 oracle (method: page "Kontekst 262K na jednej
RTX 4090: co dodałem do llama.cpp-turboq", section "Od czego zacząłem")."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from long_context_attention_tbq4_amd import _lib
from oracle import tbq4_oracle as o
from _util import check_attn

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("B,H,G,n_ctx,cap,P", [(2, 2, 8, 1000, 1024, 0), (1, 1, 4, 33, 40, 3)])
def test_c_program_decodes_on_gpu(tmp_path, B, H, G, n_ctx, cap, P):
    lib = _lib.LIB_PATH
    exe = tmp_path / "abi_gpu_decode"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_gpu_decode.c"), "-o", str(exe),
                    lib, "-Wl,-rpath," + os.path.dirname(lib),
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
    rng = np.random.default_rng(900 + n_ctx)
    seed, scale = 11, 0.09
    k = (rng.standard_t(5, size=(B, n_ctx, H, 128)) * 2.0).astype(np.float32)
    v = rng.standard_normal((B, n_ctx, H, 128)).astype(np.float32)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    for name, a in (("k.bin", k), ("v.bin", v), ("q.bin", q)):
        a.tofile(tmp_path / name)
    r = subprocess.run([str(exe), str(tmp_path), str(B), str(H), str(H * G), str(cap), str(n_ctx),
                        str(P), str(seed), repr(scale)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    kc = np.fromfile(tmp_path / "kc.bin", np.uint8).reshape(B, H, cap, 66)
    vc = np.fromfile(tmp_path / "vc.bin", np.uint8).reshape(B, H, cap, 66)
    out = np.fromfile(tmp_path / "out.bin", np.float32).reshape(B, H * G, 128)
    want_k = o.quantize_blocks(k.transpose(0, 2, 1, 3), seed)[0]
    want_v = o.quantize_blocks(v.transpose(0, 2, 1, 3), seed)[0]
    assert np.array_equal(kc[:, :, :n_ctx], want_k)
    assert np.array_equal(vc[:, :, :n_ctx], want_v)
    assert not kc[:, :, n_ctx:].any() and not vc[:, :, n_ctx:].any()
    ref = o.attn_decode_ref(q, want_k, want_v, n_ctx, np.float32(scale), seed)
    check_attn(out, ref, False, f"C program decode B={B} H={H} G={G} n_ctx={n_ctx} P={P}")
    # the decode step (prefix appended, then the last token appended and
    # attended in one call): the same bytes and the same attention bar
    kc2 = np.fromfile(tmp_path / "kc_step.bin", np.uint8).reshape(B, H, cap, 66)
    vc2 = np.fromfile(tmp_path / "vc_step.bin", np.uint8).reshape(B, H, cap, 66)
    out2 = np.fromfile(tmp_path / "out_step.bin", np.float32).reshape(B, H * G, 128)
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)
    check_attn(out2, ref, False, f"C program decode step B={B} H={H} G={G} n_ctx={n_ctx} P={P}")
