"""The host suites (block manager, scheduler, C ABI argument checks) again,
on a build of the library whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer: any out-of-bounds access, use after free or
undefined arithmetic in the host code aborts the inner run.  CPU only."""

import os
import shutil

import pytest

LLVM = "/opt/rocm/llvm"


@pytest.mark.skipif(not os.path.isdir(LLVM) or shutil.which("nm") is None,
                    reason="needs the ROCm clang and its sanitizer runtime")
def test_host_suites_clean_under_asan_and_ubsan():
    sanitize = pytest.importorskip("paged_attention_kv_cache_amd.sanitize")
    sanitize.build_sanitized(verbose=False)
    assert sanitize.run_suites() == 0
