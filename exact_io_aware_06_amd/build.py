"""Build the HIP library ``libattn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m exact_io_aware_06_amd.build`` (or call ``build()``).
The library is written next to this file; the Python binding loads it from
there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libattn.so")

SOURCES = ["attn_abi.cpp", "runtime.hip", "fwd_bf16.hip", "fwd_bf16_split.hip",
           "fwd_bf16_local.hip", "fwd_bf16_local_split.hip", "fwd_bf16_varlen.hip",
           "fwd_bf16_stream.hip",
           "fwd_f32.hip", "combine.hip", "bwd_bf16.hip", "bwd_bf16_masked.hip",
           "scratch.hip"]

# Per-source additions. The backward kernels are scheduled with the
# compiler's iterative-maxocc strategy (measured: headline backward 1.91 ->
# 1.76 ms, c3 causal backward 1.13 -> 1.09 ms); on the forward it measured
# within noise of the default and is not used.
_BWD_SCHED = ["-mllvm", "--amdgpu-sched-strategy=iterative-maxocc"]
EXTRA_FLAGS = {
    "bwd_bf16.hip": _BWD_SCHED,
    "bwd_bf16_masked.hip": _BWD_SCHED,
}

# -packed-fp32-ops: keep the compiler from emitting v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link the library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-I", INCLUDE, "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [*common, *EXTRA_FLAGS.get(src, []), "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return obj, res

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for obj, res in results:
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {obj} with exit code {res.returncode}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[obj for obj, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
