"""Compile the HIP library ``libh3attn.so`` for gfx950 with hipcc.

Run ``python -m causal_grouped_query_amd.build`` (or ``__graft_entry__.build()``).
The library is built in-tree, next to this file, so it travels with the
source tree and is the one the Python binding loads.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "h3attn.hip")]
HEADERS = [os.path.join(PKG, "csrc", n) for n in (
    "calib_kernel.hpp", "gqa_fwd_kernel.hpp", "gqa_fwd_body.inc", "gqa_fwd_wide_kernel.hpp",
    "tile_phases.inc")] + [os.path.join(ROOT, "include", "h3attn.h")]
LIBRARY = os.path.join(PKG, "libh3attn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU ops (v_pk_*_f32) stay off: plain fp32 instructions only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def build(verbose: bool = False, extra_flags=()) -> str:
    """Build ``libh3attn.so``; returns its path.  Always recompiles."""
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know this device feature
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs[:40]))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    # every symbol must resolve (a kernel whose host stub failed to instantiate would not)
    chk = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r})"],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        raise RuntimeError("built library does not load:\n" + chk.stderr[-2000:])
    os.replace(tmp, LIBRARY)
    return LIBRARY


# Host-side sanitizers for a CPU-only test build: each -fsanitize= applies to the host
# pass only (the device code is compiled as usual and never run by that test).
SANITIZE_HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-shared-libsan",
]


def build_host_sanitized(output: str) -> str:
    """Build the library with AddressSanitizer and UndefinedBehaviorSanitizer on its host
    code into ``output`` (not the in-tree library).  It needs the sanitizer runtime
    (``sanitizer_runtime()``) preloaded into the process that loads it."""
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1"] + SANITIZE_HOST_FLAGS
    cmd = [hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *SOURCES, "-o", output]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + (res.stdout + res.stderr)[-4000:])
    return output


def sanitizer_runtime() -> str | None:
    """Path of the shared AddressSanitizer runtime that matches hipcc's clang, if present."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
