"""Build libfa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

``python -m exact_attention_70_amd.build`` or ``build()`` from Python.  Every
call recompiles every source; objects go to ``_build/`` at the repository
root and the shared library to ``exact_attention_70_amd/libfa.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = os.environ.get("FA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_cache.hip"]
# Per-source extra flags.  The attention kernels never test for NaN, so they
# are built without NaN-preserving semantics; that lets max() compile to a
# single v_max/v_max3 instead of canonicalize + max.
EXTRA = {"fa_fwd.hip": ["-fno-honor-nans"], "fa_bwd.hip": ["-fno-honor-nans"]}

# Packed fp32 VALU forms are disabled for all device code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libfa needs the ROCm toolchain to build")


def _compile(src: str, verbose: bool, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-c", os.path.join(CSRC, src),
           "-o", obj] + COMMON + DEVICE_FLAGS + EXTRA.get(src, []) + list(extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link ``out``; ``defines`` are extra -D flags."""
    objdir = OBJDIR if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, objdir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", flush=True)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
