"""Full-size workloads against the fp64 oracle, in the launch configuration the benchmark
times (needs a gfx950 GPU).

The S=10231 and S=7680 text-encoder workloads are compared over their whole outputs: every
query token and head of O (relative L2 and max |error| over the whole tensor) and of LSE.
The larger workloads (the packed T=35124 batch, the S=32768 stress workload and the two
DiT sizes) are compared on one query token of every 32-token query block, its offset in
the block moving with the block index (position 32 b + (b mod 32)), every head; the
oracle on all of their rows takes minutes each on the host, too long for a GPU test run.
"""

from __future__ import annotations

import time

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import causal_grouped_query_amd as h3

    h3.load_library()
    return h3


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield


def _causal(h3, w, inp):
    import torch

    q, k, v = (to_device(inp[n]) for n in ("q", "k", "v"))
    if w.varlen:
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
        o, lse = h3.gqa_causal_varlen_fwd(q, k, v, cu, max(w.seqlens), softmax_scale=w.scale)
    else:
        o, lse = h3.gqa_causal_fwd(q, k, v, softmax_scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


def _oracle(w, inp, tokens):
    t0 = time.perf_counter()
    n = w.total_tokens if tokens is None else len(tokens)
    print(f"[gpu-test] oracle on {n} query tokens x {w.n_q_heads} heads "
          f"({oracle.threads()} threads)", flush=True)
    if w.causal:
        ref = oracle.gqa_causal_varlen(inp["q"], inp["k"], inp["v"], w.cu_seqlens, w.scale,
                                       tokens=tokens)
    else:
        ref = oracle.gqa_bidirectional(inp["q"], inp["k"], inp["v"], w.scale, tokens=tokens)
    print(f"[gpu-test] oracle done in {time.perf_counter() - t0:.1f} s", flush=True)
    return ref


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["under_cap_s7680", "failing_s10231"])
def test_whole_output(lib, name):
    w = workloads.ALL_WORKLOADS[name]
    inp = workloads.generate(w)
    o, lse = _causal(lib, w, inp)
    o_gpu, lse_gpu = to_f64(o), to_f64(lse)
    del o, lse
    o_ref, lse_ref = _oracle(w, inp, None)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    assert_close(o_gpu, lse_gpu, o_ref, lse_ref, f"{name}, whole O and LSE")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["varlen_4x_t35124", "stress_s32768"])
def test_causal_every_query_block(lib, name):
    import torch

    w = workloads.ALL_WORKLOADS[name]
    inp = workloads.generate(w)
    o, lse = _causal(lib, w, inp)
    tokens = workloads.block_tokens(w.seqlens)
    assert len(tokens) == sum((s + 31) // 32 for s in w.seqlens)
    o_ref, lse_ref = _oracle(w, inp, tokens)
    idx = torch.from_numpy(tokens).cuda()
    assert_close(to_f64(o.index_select(0, idx)), to_f64(lse.index_select(1, idx)), o_ref,
                 lse_ref, f"{name}, one token of each of {len(tokens)} query blocks")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dit_s19316_h32_d128", "dit_s34121_h32_d128"])
def test_bidirectional_every_query_block(lib, name):
    import torch

    w = workloads.ALL_WORKLOADS[name]
    inp = workloads.generate(w)
    q, k, v = (to_device(inp[n]) for n in ("q", "k", "v"))
    o, lse = lib.gqa_fwd(q, k, v, causal=False, softmax_scale=w.scale)     # token-major O
    torch.cuda.synchronize()
    tokens = workloads.block_tokens(w.seqlens)
    o_ref, lse_ref = _oracle(w, inp, tokens)
    idx = torch.from_numpy(tokens).cuda()
    assert_close(to_f64(o.index_select(0, idx)), to_f64(lse.index_select(1, idx)), o_ref,
                 lse_ref, f"{name}, one token of each of {len(tokens)} query blocks")
