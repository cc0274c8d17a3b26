"""Q/K prologue (RMS norm + RoPE) against the fp64 oracle, through the C ABI entry
h3attn_qk_norm_rope (needs a gfx950 GPU).

Bound per element: the kernel computes in fp32 and rounds each output to bf16 once, so
|gpu - exact| <= 2^-8 |exact| (bf16 rounding, with margin) + 2^-16 * the row's RMS (fp32
arithmetic and cancellation in the rotation).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, bits_of, to_device, to_f64
from workloads import f32_to_bf16_bits, normal_inputs

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


def _check(gpu_bits, ref, what):
    g = workloads.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
    err = np.abs(g - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * rms
    worst = float((err / np.maximum(bound, 1e-300)).max())
    print(f"[prologue] {what}: max err {err.max():.3e}, worst err/bound {worst:.3f}", flush=True)
    assert np.all(np.isfinite(g)), what
    assert np.all(err <= bound), what


def _weights(seed, D):
    w = np.random.Generator(np.random.PCG64(seed)).uniform(0.5, 1.5, D).astype(np.float32)
    return f32_to_bf16_bits(w)


CASES = [  # S, Hq, Hkv, D, seed, norm, rope, explicit positions
    (1, 8, 2, 128, 601, True, True, False),
    (37, 8, 2, 128, 602, True, True, False),
    (100, 16, 16, 64, 603, True, True, True),
    (257, 64, 8, 128, 604, False, True, False),
    (64, 4, 1, 64, 605, True, False, False),
    (333, 32, 4, 128, 606, True, True, True),
]


@pytest.mark.parametrize("S,Hq,Hkv,D,seed,norm,rope,explicit", CASES)
def test_prologue_small(lib, S, Hq, Hkv, D, seed, norm, rope, explicit):
    import torch

    q, k, _ = normal_inputs(seed, S, Hq, Hkv, D, sigma=2.0)
    wq, wk = _weights(seed + 1, D), _weights(seed + 2, D)
    pos = (np.random.Generator(np.random.PCG64(seed + 3)).integers(0, 40000, S)
           if explicit else None)
    theta = 1e6 if D == 128 else 1e4
    qo, ko = lib.qk_norm_rope(
        to_device(q), to_device(k), to_device(wq) if norm else None,
        to_device(wk) if norm else None, eps=1e-6, rope=rope, rope_theta=theta,
        positions=torch.from_numpy(pos.astype(np.int32)).cuda() if explicit else None)
    torch.cuda.synchronize()
    rq = oracle.qk_norm_rope(q, weight=wq if norm else None, eps=1e-6, rope=rope, theta=theta,
                             positions=pos)
    rk = oracle.qk_norm_rope(k, weight=wk if norm else None, eps=1e-6, rope=rope, theta=theta,
                             positions=pos)
    _check(bits_of(qo), rq, f"q S={S} Hq={Hq} D={D} norm={norm} rope={rope}")
    _check(bits_of(ko), rk, f"k S={S} Hkv={Hkv} D={D} norm={norm} rope={rope}")


def test_prologue_in_place(lib):
    """Writing over the inputs gives the same bits as writing to new tensors."""
    import torch

    S, Hq, Hkv, D = 300, 16, 4, 128
    q, k, _ = normal_inputs(610, S, Hq, Hkv, D)
    wq, wk = to_device(_weights(611, D)), to_device(_weights(612, D))
    qd, kd = to_device(q), to_device(k)
    qo, ko = lib.qk_norm_rope(qd, kd, wq, wk)
    lib.qk_norm_rope(qd, kd, wq, wk, q_out=qd, k_out=kd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(qo), bits_of(qd))
    assert np.array_equal(bits_of(ko), bits_of(kd))


def test_prologue_primary_size(lib):
    """The primary workload's Q and K (S=10231, 64/8 heads, D=128), norm + RoPE, every
    element against the oracle."""
    import torch

    w = workloads.WORKLOADS[workloads.PRIMARY]
    inp = workloads.generate(w)
    wq, wk = _weights(620, 128), _weights(621, 128)
    qo, ko = lib.qk_norm_rope(to_device(inp["q"]), to_device(inp["k"]), to_device(wq),
                              to_device(wk))
    torch.cuda.synchronize()
    _check(bits_of(qo), oracle.qk_norm_rope(inp["q"], weight=wq), "q primary")
    _check(bits_of(ko), oracle.qk_norm_rope(inp["k"], weight=wk), "k primary")


def test_prologue_then_attention(lib):
    """Prologue then attention on the GPU against the oracle's prologue (rounded to bf16)
    then the oracle's attention."""
    import torch

    S, Hq, Hkv, D = 700, 16, 2, 128
    q, k, v = normal_inputs(630, S, Hq, Hkv, D)
    wq, wk = _weights(631, D), _weights(632, D)
    qo, ko = lib.qk_norm_rope(to_device(q), to_device(k), to_device(wq), to_device(wk))
    scale = workloads.default_scale(D)
    o, lse = lib.gqa_causal_fwd(qo, ko, to_device(v), softmax_scale=scale)
    torch.cuda.synchronize()
    rq = f32_to_bf16_bits(oracle.qk_norm_rope(q, weight=wq).astype(np.float32))
    rk = f32_to_bf16_bits(oracle.qk_norm_rope(k, weight=wk).astype(np.float32))
    o_ref, lse_ref = oracle.gqa_causal(rq, rk, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, "prologue + attention")
