"""Builds libkq.so (the C-ABI library of HIP kernels) in-tree for gfx950.

    python -m post_quantization_03_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkq.so")
PROBE_LIB = os.path.join(HERE, "libkqprobe.so")
SOURCES = ("api", "dense", "gj", "syrk", "hadamard", "sweep", "dequant", "hgprep")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wno-unused-result", "-Wno-unused-value",
         "-Wno-pass-failed", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str) -> str:
    out = os.path.join(OBJ, src + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src + ".hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}.hip:\n{r.stderr[-4000:]}")
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    # the throughput probes of the execution units and HBM: a library of their own, outside the C ABI
    pobj = _compile("probe")
    ptmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", ptmp, pobj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stderr[-4000:]}")
    os.replace(ptmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
