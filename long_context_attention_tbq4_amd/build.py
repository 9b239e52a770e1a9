"""Build libtbq4.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m long_context_attention_tbq4_amd.build

Every HIP source under csrc/ is compiled for gfx950 only and linked into one
shared object next to this file.  Packed-FP32 instruction selection is
disabled on the device side (-packed-fp32-ops) as a deliberate choice for
numerical robustness.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libtbq4.so")
SOURCES = ["api.cpp", "quantize.hip", "decode.hip", "verify.hip", "prefill.hip",
           "bench_kernels.hip"]
# per-source options: the decode and verify loops keep their MFMA
# accumulators in ordinary VGPRs (the conditional rescale and the scores then
# need no copies between accumulation and vector registers)
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "verify.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    """Compile every source and link libtbq4.so; returns the library path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-function"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = ([hipcc()] + common + EXTRA.get(src, []) +
               ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc(), "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err:
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
