"""Compile the plain-C consumer of the C ABI (c_consumer.c) into libc_consumer.so, next to
its source.  Test infrastructure: the GPU test tests/test_gpu_c_consumer.py loads it."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "c_consumer.c")
LIBRARY = os.path.join(HERE, "libc_consumer.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(output: str, werror: bool = False) -> list:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("c_consumer: no C compiler (gcc) found")
    return [cc, "-std=c11", "-O2", "-Wall", "-Wextra", *(["-Werror"] if werror else []),
            "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
            f"-I{os.path.join(ROOT, 'include')}", SOURCE, "-o", output, "-ldl",
            f"-L{ROCM}/lib", "-lamdhip64", "-lm"]


def build(output: str = LIBRARY) -> str:
    tmp = output + ".tmp"
    subprocess.run(command(tmp), check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
