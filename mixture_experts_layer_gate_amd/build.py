"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: ``python -m mixture_experts_layer_gate_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "route.hip", "permute.hip", "combine.hip", "ffn_f32.hip", "ffn_bf16.hip",
           "ffn_fp8.hip", "ffn_fp4.hip", "quant.hip", "balance.hip", "backward.hip", "backward_fp8.hip", "wgrad.hip"]
# measurement tooling for the benchmark's roofline figures, in a library of its own (not libmoe.so)
PROBE_SOURCES = ["peak_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # no packed fp32 instructions in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]

# Per-source extra flags. The fp8 GEMMs scale their MFMA accumulators on the
# VALU between K chunks, so the accumulators must be MFMA destinations in
# VGPRs (left to itself the compiler keeps them in AGPRs and copies every
# element out and back for each multiply).
EXTRA = {"ffn_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "ffn_fp4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
