"""The header include/h3attn.h compiles as C (C11, every warning an error) in the plain-C
consumer of the C ABI that the GPU tests run; no GPU involved."""

from __future__ import annotations

import importlib.util
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def _builder():
    spec = importlib.util.spec_from_file_location(
        "build_consumer", os.path.join(HERE, "c_consumer", "build_consumer.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_consumer_compiles_as_c_with_warnings_as_errors(tmp_path):
    b = _builder()
    out = tmp_path / "libc_consumer.so"
    r = subprocess.run(b.command(str(out), werror=True), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    nm = subprocess.run(["nm", "-D", "--defined-only", str(out)], capture_output=True, text=True)
    assert "h3attn_c_consumer_run" in nm.stdout
