"""Build libyrb.so (HIP for gfx950) in-tree with hipcc.

    python -m yarn_rope_blockwise_amd.build

Compiles every source under csrc/ to an object (in parallel), links them
into ``yarn_rope_blockwise_amd/libyrb.so`` and replaces the old library
atomically.  Cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libyrb.so")
SOURCES = ["api.cpp", "rope.hip", "attn.hip", "attn_pp.hip", "decode.hip", "noalloc.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code; the compiler
# still emits ordinary scalar fp32 and the MFMA/DS/LDS-DMA instructions.
FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, build_dir: str = BUILD, extra=(), csrc: str = CSRC) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-I", CSRC, "-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = [ln for ln in r.stderr.splitlines()
            if "warning" in ln and "packed-fp32-ops" not in ln]
    if warn:
        sys.stderr.write(f"[yrb build] {src}:\n" + "\n".join(warn) + "\n")
    return obj


def build(verbose: bool = True, lib: str = LIB, build_dir: str = BUILD, extra=(),
          csrc: str = CSRC) -> str:
    """Compile and link.  ``extra`` flags, ``csrc`` and the output path allow
    building variants of the library elsewhere."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra, csrc), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"[yrb build] {lib}")
    return lib


if __name__ == "__main__":
    build()
