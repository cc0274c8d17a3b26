"""The C ABI from plain C (needs a gfx950 GPU): tests/c_consumer/c_consumer.c allocates device
buffers with the HIP runtime, resolves the library's entry points by name, runs a fixed-length
call at D = 128 and D = 64 and a packed call with an empty sequence, checks them against the
fp64 oracle and checks that rejected calls return their status and write nothing.  Its shared
object is built by the repository's build step; it runs in this process, after torch, so it
uses the same HIP runtime."""

from __future__ import annotations

import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CONSUMER = os.path.join(HERE, "c_consumer", "libc_consumer.so")


def test_plain_c_caller():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import causal_grouped_query_amd as h3
    import oracle

    h3.load_library()
    oracle.default()                          # the oracle's shared object is built and loads
    assert os.path.exists(CONSUMER), "build the repository first (__graft_entry__.build())"
    print(f"\n[gpu-test] plain-C consumer {CONSUMER}", flush=True)
    lib = ctypes.CDLL(CONSUMER)
    lib.h3attn_c_consumer_run.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p,
                                          ctypes.c_int]
    lib.h3attn_c_consumer_run.restype = ctypes.c_int
    report = ctypes.create_string_buffer(8192)
    rc = lib.h3attn_c_consumer_run(h3.LIBRARY.encode(), oracle.LIBRARY.encode(), report, 8192)
    text = report.value.decode()
    print(text, flush=True)
    assert rc == 0, text
    assert text.count(" ok") == 7, text       # three calls, four rejections
