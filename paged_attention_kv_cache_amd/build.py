"""Build ``libpagedattn.so`` for gfx950 with hipcc, in-tree.

Each source compiles to its own object in ``_build/`` (in parallel), then
one link step writes the shared library next to this file.  Every build
recompiles everything: the build is the "does it compile" check.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["abi.cpp", "kv_cache_write.hip", "pa_decode.hip", "pa_prefill.hip", "kv_manager.cpp", "stream_read.hip",
           "serve.cpp"]
# plain host C++ (no device code): built by the host compiler
HOST_SOURCES = {"kv_manager.cpp"}
# per-source device flags.  The prefill kernel never relies on NaN semantics
# (masked and poisoned keys are removed by selects on integer conditions and
# zeroed V rows), so it runs without the IEEE-mode NaN quieting, which would
# otherwise add a canonicalising move before every max of an MFMA result.
SOURCE_FLAGS = {"pa_prefill.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # keep packed fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, extra: list[str], build_dir: str = BUILD, host_cxx: str | None = None,
             host_extra: list[str] | None = None) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    if src in HOST_SOURCES:
        cmd = [host_cxx or os.environ.get("CXX", "g++"), *HOST_FLAGS, *(host_extra or []),
               "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None, out_path: str | None = None,
          build_dir: str | None = None, host_cxx: str | None = None, host_extra: list[str] | None = None,
          link_extra: list[str] | None = None) -> str:
    """Compile every source and link the library (default: in-tree next to
    this file).  ``extra_flags`` go to every hipcc compile, e.g.
    ``-DNAME=value``; ``host_cxx`` / ``host_extra`` replace the compiler of
    the plain C++ sources and add flags to it; ``link_extra`` goes to the
    link step."""
    bdir = build_dir or BUILD
    out = out_path or LIB_PATH
    os.makedirs(bdir, exist_ok=True)
    extra = list(extra_flags or [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, bdir, host_cxx, host_extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *(link_extra or []), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
