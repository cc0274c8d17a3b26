"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with both sanitizers on its host pass (the device code is compiled as
usual and never launched here) and the C-ABI tests that need no GPU -- every rejection case
of every entry point, the no-op calls, the offsets check, the size queries and status
strings -- run against it in a child process with the sanitizer runtime preloaded.  Any
sanitizer report fails the child and this test.
"""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

from causal_grouped_query_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# test_abi tests that read the library's code object (kernel metadata, instructions) are
# about the production build's device code, not its host code: left out here
CODE_OBJECT_TESTS = ("lds_bytes_fixed", "kernel_lds", "packed_fp32", "lds_dma")


@pytest.mark.timeout(900)
def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    rt = hip_build.sanitizer_runtime()
    assert rt, "no AddressSanitizer runtime next to hipcc's clang"
    lib = hip_build.build_host_sanitized(str(tmp_path / "libh3attn_sanitized.so"))
    env = dict(os.environ, LD_PRELOAD=rt, H3ATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    select = " and ".join(f"not {t}" for t in CODE_OBJECT_TESTS)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi.py"), "-k", select],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    print(out)
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout
