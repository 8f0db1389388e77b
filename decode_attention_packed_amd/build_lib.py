"""Builds libkvq.so (the HIP library behind include/kvq.h) for gfx950 in-tree.

Each source is compiled with hipcc into _build/ in parallel, then linked
into decode_attention_packed_amd/libkvq.so.  Packed fp32 VALU instructions
are disabled on the device pass (-packed-fp32-ops); the host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kvq_api.cpp", "kvq_append.hip", "kvq_attn.hip", "kvq_attn_f16k.hip", "kvq_attn_w12.hip",
           "kvq_debug.hip"]
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA accumulators in VGPRs (no AGPR copies around each MFMA)
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          # inputs are finite by contract: max/min need no NaN quieting
          "-fno-honor-nans",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source and link libkvq.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
