"""Build libzgattn.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m global_causal_attention_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libzgattn.so")
SOURCES = ["prefill.hip", "prefill_swa.hip", "decode.hip", "stack.hip", "stack_fp8.hip", "backward.hip",
           "probe.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function",
         # no packed-fp32 VALU instructions in any kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source additions. backward.hip: matrix products whose results the vector units read land in
# ordinary VGPRs (bwd_kv keeps its long-lived dV/dK sums in AGPRs through asm-form MFMAs).
EXTRA_FLAGS = {"backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    inc = ["-I", os.path.join(os.path.dirname(PKG), "include")]
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory() as td:
        objs = [os.path.join(td, s + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, *EXTRA_FLAGS.get(s, []), *inc, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
