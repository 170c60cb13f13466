"""Host sanitizer build: AddressSanitizer + UndefinedBehaviorSanitizer on
the host code of the library (the C ABI's argument checks, the KV block
manager and the step scheduler), with the host test suites run on it.

Only the host side is instrumented (every sanitizer flag goes through
``-Xarch_host``; the gfx950 code objects are built exactly as in the
normal build).  The plain C++ sources are compiled by the ROCm clang so
that one sanitizer runtime (clang's) serves every object; the Python
interpreter is not instrumented, so that runtime is preloaded.  The host
suites issue no GPU work, so this runs on a machine without a GPU.

    python -m paged_attention_kv_cache_amd.sanitize            # build + run
    python -m paged_attention_kv_cache_amd.sanitize --no-build # run only

Leak checking is off: the interpreter and torch keep allocations alive
until exit by design, which would bury any report from this library.
"""

from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys

from . import build as B

SAN_BUILD = os.path.join(B.PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libpagedattn_san.so")
LLVM = "/opt/rocm/llvm"
SUITES = ["tests/test_kv_manager.py", "tests/test_abi_host.py"]
_CHECKS = ["address", "undefined"]


def _host_only(flags: list[str]) -> list[str]:
    out: list[str] = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def san_flags() -> list[str]:
    return _host_only([f"-fsanitize={c}" for c in _CHECKS] +
                      ["-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"])


def runtime() -> str:
    cands = sorted(glob.glob(os.path.join(LLVM, "lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")))
    if not cands:
        raise RuntimeError(f"no clang AddressSanitizer runtime under {LLVM}")
    return cands[-1]


def build_sanitized(verbose: bool = True) -> str:
    flags = san_flags()
    return B.build(verbose=verbose, extra_flags=flags, out_path=SAN_LIB, build_dir=SAN_BUILD,
                   host_cxx=os.path.join(LLVM, "bin/clang++"), host_extra=flags,
                   link_extra=flags + ["-shared-libasan"])


def run_suites(extra_args: list[str] | None = None) -> int:
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime()
    env["PA_LIBRARY"] = SAN_LIB
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1:check_initialization_order=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *SUITES, *(extra_args or [])]
    return subprocess.run(cmd, cwd=B.ROOT, env=env).returncode


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--no-build", action="store_true", help="reuse the sanitized library already built")
    args, rest = ap.parse_known_args()
    if not args.no_build:
        build_sanitized()
    return run_suites(rest)


if __name__ == "__main__":
    sys.exit(main())
