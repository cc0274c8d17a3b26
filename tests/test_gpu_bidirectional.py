"""Bidirectional (non-causal) path and the head-major output layout against the fp64
oracle, through the C ABI entry h3attn_gqa_fwd (needs a gfx950 GPU)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, bits_of, to_device, to_f64
from workloads import DIT_WORKLOADS, normal_inputs, stress_inputs

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


def _bi(h3, q, k, v, scale, head_major=False):
    import torch

    o, lse = h3.gqa_fwd(to_device(q), to_device(k), to_device(v), causal=False,
                        head_major_out=head_major, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


SMALL = [  # S, Hq, Hkv, D, seed: every group size and head dim, ragged lengths
    (1, 8, 8, 128, 401),
    (63, 8, 2, 64, 402),
    (64, 16, 16, 128, 403),
    (65, 4, 4, 64, 404),
    (200, 16, 2, 128, 405),
    (333, 32, 32, 128, 406),
    (517, 8, 1, 64, 407),
    (1000, 16, 4, 128, 408),
]


@pytest.mark.parametrize("S,Hq,Hkv,D,seed", SMALL)
def test_bidirectional_small_full_parity(lib, S, Hq, Hkv, D, seed):
    q, k, v = normal_inputs(seed, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    o, lse = _bi(lib, q, k, v, scale)
    o_ref, lse_ref = oracle.gqa_bidirectional(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref,
                 f"bidirectional S={S} Hq={Hq} Hkv={Hkv} D={D}")


def test_bidirectional_large_logits(lib):
    q, k, v, _ = stress_inputs(410, 777, 16, 2, 128)
    scale = workloads.default_scale(128)
    o, lse = _bi(lib, q, k, v, scale)
    o_ref, lse_ref = oracle.gqa_bidirectional(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, "bidirectional stress S=777")


@pytest.mark.parametrize("causal", [True, False])
def test_head_major_is_token_major_transposed(lib, causal):
    """O written [Hq, S, D] holds the same bits as the [S, Hq, D] result, transposed."""
    import torch

    S, Hq, Hkv, D = 300, 16, 4, 128
    q, k, v = normal_inputs(420, S, Hq, Hkv, D)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o_t, l_t = lib.gqa_fwd(qd, kd, vd, causal=causal)
    o_h, l_h = lib.gqa_fwd(qd, kd, vd, causal=causal, head_major_out=True)
    torch.cuda.synchronize()
    assert o_h.shape == (Hq, S, D)
    assert np.array_equal(bits_of(o_h), bits_of(o_t.transpose(0, 1).contiguous()))
    assert torch.equal(l_h, l_t)


def test_flags_zero_is_the_causal_call(lib):
    """h3attn_gqa_fwd with no flags is bit-identical to h3attn_gqa_causal_fwd."""
    import torch

    S, Hq, Hkv, D = 257, 8, 2, 64
    q, k, v = normal_inputs(430, S, Hq, Hkv, D)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o1, l1 = lib.gqa_fwd(qd, kd, vd)
    o2, l2 = lib.gqa_causal_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(o1), bits_of(o2))
    assert torch.equal(l1, l2)


def test_bidirectional_key_permutation(lib):
    """Permuting the K/V rows together leaves the result unchanged up to rounding."""
    S, Hq, Hkv, D = 400, 8, 2, 128
    q, k, v = normal_inputs(440, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    o1, l1 = _bi(lib, q, k, v, scale)
    perm = np.random.Generator(np.random.PCG64(441)).permutation(S)
    o2, l2 = _bi(lib, q, k[perm], v[perm], scale)
    assert_close(to_f64(o2), to_f64(l2), to_f64(o1), to_f64(l1), "key permutation")


@pytest.mark.parametrize("name", sorted(DIT_WORKLOADS))
def test_dit_workload_sampled(lib, name):
    """The DiT-size workloads at full size: sampled query tokens (every head) against the
    oracle, in the launch configuration the benchmark times, head-major output."""
    import torch

    w = DIT_WORKLOADS[name]
    inp = workloads.generate(w)
    q, k, v = (to_device(inp[n]) for n in ("q", "k", "v"))
    o, lse = lib.gqa_fwd(q, k, v, causal=False, head_major_out=True, softmax_scale=w.scale)
    torch.cuda.synchronize()
    tokens = workloads.sample_tokens(w.seqlens, 12, seed=w.seed + 700)
    o_ref, lse_ref = oracle.gqa_bidirectional(inp["q"], inp["k"], inp["v"], w.scale,
                                              tokens=tokens)
    idx = torch.from_numpy(tokens).cuda()
    o_s = o.transpose(0, 1).index_select(0, idx)
    assert_close(to_f64(o_s), to_f64(lse.index_select(1, idx)), o_ref, lse_ref,
                 f"{name} (sampled)")
