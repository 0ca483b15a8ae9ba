"""Build libxr.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python cross_entropy_reductions_amd/build.py`` (run by path: importing the package
needs the library this builds), or ``__graft_entry__.build()``. The library lands next to
this file as ``libxr.so``; nothing is installed elsewhere.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libxr.so")
SOURCES = ["xr_xent.hip", "xr_softmax.hip", "xr_layernorm.hip", "xr_bsr.hip", "xr_noalloc.hip",
           "xr_probe.hip", "xr_api.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set HIPCC or install ROCm")


def build(verbose: bool = False, output: str = LIBRARY, defines=()) -> str:
    """Compile every source and link libxr.so; always rebuilds. Returns the library path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="xr_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [cc, *HIPCC_FLAGS, *(f"-D{d}" for d in defines), "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
            return obj

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp_out = output + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(tmp_out, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
