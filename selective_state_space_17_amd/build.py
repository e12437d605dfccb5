"""Build libmssm.so (HIP for gfx950) in-tree.

    python selective_state_space_17_amd/build.py

(run as a script: importing the package would open the library being rebuilt)

hipcc compiles for gfx950 only.  Packed-fp32 VALU instructions are disabled
(-packed-fp32-ops); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmssm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.cpp", "scan_m1.hip", "ssd_m2.hip", "decode.hip", "bwd_m1.hip", "noalloc.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wno-inline-asm",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared",)] + ["-c"] + lang + \
          ["-I", os.path.join(ROOT, "include"), "-o", obj, os.path.join(CSRC, src)]
    subprocess.check_call(cmd, stderr=subprocess.STDOUT)


def build(verbose: bool = True) -> str:
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    t = time.time()
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
