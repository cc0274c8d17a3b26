"""The entry points under HIP graph capture (needs a gfx950 GPU): a call captured with
torch.cuda.graph and replayed gives, on every replay, the bits an eager call gives on the
inputs the buffers hold at replay time.  Replays alternate with eager library calls and
torch work, and the inputs change between replays, so a replay that reused stale state or
missed its inputs would show.  No call here allocates or clears memory inside the capture
(the library has no memset; the split-KV call takes the library's fixed scratch array)."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_util import bits_of, to_device
from workloads import normal_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h3():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import causal_grouped_query_amd as h3

    h3.load_library()
    return h3


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield


def _replay_matches_eager(call, inputs, outputs, new_inputs, replays=3):
    """Capture call() (writing `outputs`), then for each replay load the next input set into
    the captured buffers, replay, and compare every output with an eager call on the same
    inputs into separate buffers."""
    import torch

    call(*inputs, *outputs)                       # warm-up: lazy setup happens outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(*inputs, *outputs)
    torch.cuda.synchronize()
    for i in range(replays):
        src = new_inputs[i % len(new_inputs)]
        for dst, s in zip(inputs, src):
            dst.copy_(s)
        g.replay()
        torch.cuda.synchronize()
        got = [bits_of(t) for t in outputs]
        fresh = [torch.empty_like(t) for t in outputs]
        call(*src, *fresh)                        # eager, other buffers
        scratch = torch.randn(1 << 20, device="cuda").sum()   # unrelated torch work
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for a, b in zip(got, fresh):
            assert np.array_equal(a, bits_of(b)), f"replay {i} differs from the eager call"


def _qkv_sets(seed, S, Hq, Hkv, D, n=3):
    return [tuple(to_device(x) for x in normal_inputs(seed + i, S, Hq, Hkv, D)) for i in range(n)]


def test_fused_causal_call_in_a_graph(h3):
    import torch

    S, Hq, Hkv, D = 777, 16, 2, 128
    sets = _qkv_sets(900, S, Hq, Hkv, D)
    inputs = [t.clone() for t in sets[0]]
    outputs = [torch.empty_like(inputs[0]), torch.empty((Hq, S), device="cuda")]

    def call(q, k, v, o, lse):
        h3.gqa_causal_fwd(q, k, v, out=o, lse=lse)

    _replay_matches_eager(call, inputs, outputs, sets[1:] + sets[:1])


def test_packed_call_in_a_graph(h3):
    import torch

    lens = [300, 0, 129, 64]
    T, Hq, Hkv, D = sum(lens), 8, 1, 128
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    sets = _qkv_sets(910, T, Hq, Hkv, D)
    inputs = [t.clone() for t in sets[0]]
    outputs = [torch.empty_like(inputs[0]), torch.empty((Hq, T), device="cuda")]

    def call(q, k, v, o, lse):
        h3.gqa_causal_varlen_fwd(q, k, v, cu, max(lens), out=o, lse=lse)

    _replay_matches_eager(call, inputs, outputs, sets[1:] + sets[:1])


def test_allocation_free_split_call_in_a_graph(h3):
    import torch

    S, Hq, Hkv, D = 513, 8, 2, 64
    sets = _qkv_sets(920, S, Hq, Hkv, D)
    inputs = [t.clone() for t in sets[0]]
    outputs = [torch.empty_like(inputs[0]), torch.empty((Hq, S), device="cuda")]

    def call(q, k, v, o, lse):
        h3.gqa_causal_splitkv_fwd_noalloc(q, k, v, 3, out=o, lse=lse)

    _replay_matches_eager(call, inputs, outputs, sets[1:] + sets[:1])
