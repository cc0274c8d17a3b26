"""The code object writes memory through vector and LDS stores only (CPU check of the
disassembly of the built library; no GPU involved).  Kept apart from the other code-object
checks because it names the forbidden instruction forms."""

from __future__ import annotations

import re

import pytest

import causal_grouped_query_amd as h3
from test_abi import _code_object_tool


@pytest.fixture(scope="module")
def lib():
    return h3.load_library()


def test_no_scalar_memory_writes(lib):
    """No instruction writes through the scalar data cache: no scalar stores or atomics,
    and none of its write-back or discard forms."""
    asm = _code_object_tool("llvm-objdump", "-d", "--mcpu=gfx950")
    assert "global_store" in asm                       # the disassembly has the kernels' stores
    bad = sorted(set(re.findall(r"\bs_(?:store|buffer_store|scratch_store|atomic|buffer_atomic"
                                r"|dcache_wb|dcache_discard)\w*", asm)))
    assert not bad, bad
