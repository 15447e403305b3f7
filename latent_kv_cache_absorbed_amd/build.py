"""Build the gfx950 shared library in-tree: ``python -m latent_kv_cache_absorbed_amd.build``.

Compiles every source under csrc/ with hipcc for gfx950 and links
``liblatent_decode.so`` next to this file.  Object files go to ``_build/`` at
the repository root.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblatent_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "plan_combine.hip", "decode.hip", "decode_pipe.hip", "decode_pipe_fp8.hip", "append.hip",
           "projection.hip", "noalloc.hip"]

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
          # packed fp32 VALU forms are kept out of every kernel
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]
# Per-source flags: the decode kernels keep the results of their builtin MFMAs in the VGPR file (at two
# waves per SIMD this avoids AGPR round trips and spills; the pipelined kernel's own P.V accumulators
# sit in AGPRs through inline asm).
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_pipe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_pipe_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def build(extra_flags=(), jobs: int = 4) -> str:
    """Compile all sources and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = sys.argv[1:]
    print(build(extra))
