"""The allocation-free split-KV entry point against the workspace one, through the C ABI
(needs a gfx950 GPU)."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, bits_of, to_device, to_f64
from workloads import normal_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import causal_grouped_query_amd as h3

    h3.load_library()
    return h3


def test_noalloc_matches_the_workspace_call_twice(lib):
    """Two calls in a row, the second with a smaller input: each gives the same bits as
    the workspace call of the same arguments, and matches the oracle."""
    import torch

    c = lib.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for S, Hq, Hkv, D, splits, seed in ((3000, 8, 1, 128, 4, 901), (333, 16, 2, 64, 3, 902)):
        print(f"[gpu-test] no-alloc split-KV S={S} Hq={Hq} Hkv={Hkv} D={D} splits={splits}",
              flush=True)
        need = lib.splitkv_workspace_bytes(S, Hq, D, splits)
        assert 0 < need <= lib.NOALLOC_SCRATCH_BYTES
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D)
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        scale = workloads.default_scale(D)
        o_ws, l_ws = lib.gqa_causal_splitkv_fwd(qd, kd, vd, splits, softmax_scale=scale)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((Hq, S), float("nan"), dtype=torch.float32, device="cuda")
        rc = c.h3attn_gqa_causal_splitkv_fwd_noalloc(
            qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), S, Hq,
            Hkv, D, ctypes.c_float(scale), splits, ctypes.c_void_p(stream))
        assert rc == lib.OK, lib.status_string(rc)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(o), bits_of(o_ws)), "O differs from the workspace call"
        assert np.array_equal(to_f64(lse), to_f64(l_ws)), "LSE differs from the workspace call"
        o_ref, lse_ref = oracle.gqa_causal(q, k, v, scale)
        assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, f"no-alloc S={S}")


def test_noalloc_refuses_a_request_past_its_scratch(lib):
    import torch

    S, Hq, Hkv, D, splits = 4096, 64, 8, 128, 2      # 2 * 4096 * 64 * 128 * 4 B = 256 MiB
    assert lib.splitkv_workspace_bytes(S, Hq, D, splits) > lib.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    with pytest.raises(lib.H3AttnError) as err:
        lib.gqa_causal_splitkv_fwd_noalloc(q, kv, kv, splits, out=o)
    assert err.value.status == lib.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()), "a refused call wrote its output"
