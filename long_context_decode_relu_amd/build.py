"""Build libssa.so (the HIP library behind the C ABI) for gfx950, in-tree.

Usage: python -m long_context_decode_relu_amd.build  (or call build()).
Each source is compiled to an object in parallel, then linked into
long_context_decode_relu_amd/libssa.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssa.so")
SOURCES = ["api.cpp", "decode_full.hip", "select.hip", "decode_sparse.hip", "prefill.hip", "cache.hip", "mlp.hip", "window.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags(src: str) -> list[str]:
    f = ["-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}"]
    if src.endswith(".hip"):
        # Packed fp32 math (v_pk_*_f32) is turned off for all device code.
        f += ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops"]
    else:
        f += ["-D__HIP_PLATFORM_AMD__"]
    return f


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _check_resolved(path: str) -> None:
    """Load the library with every symbol bound now (no GPU needed): a kernel
    whose host stub the compiler silently dropped shows up here as an
    undefined symbol instead of at the first call."""
    try:
        ctypes.CDLL(os.path.abspath(path), mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        raise RuntimeError(f"{path} does not load: {e}") from None


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    _check_resolved(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
