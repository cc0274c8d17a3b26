"""Causal GQA forward with the Q prologue (RMS norm + RoPE) inside the attention kernel,
h3attn_gqa_causal_qnorm_rope_fwd, against the fp64 oracle (needs a gfx950 GPU).

Reference: the oracle's prologue of Q and of K, each rounded to bf16 (the prologue's
output type), then the oracle's causal attention.  The GPU side transforms K with the
K-only prologue call and Q inside the attention kernel.  The kernel's Q may differ from the
rounded oracle Q by one bf16 step in a few elements (fp32 vs fp64 arithmetic), which
stays far inside the attention tolerances.
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


def _weights(seed, D):
    w = np.random.Generator(np.random.PCG64(seed)).uniform(0.5, 1.5, D).astype(np.float32)
    return f32_to_bf16_bits(w)


def _prologue_ref(x, w, rope, positions):
    return f32_to_bf16_bits(oracle.qk_norm_rope(x, weight=w, rope=rope, theta=1e6,
                                                positions=positions).astype(np.float32))


def _run(h3, q, k, v, wq, wk, rope, positions, scale):
    import torch

    pos_dev = None if positions is None else torch.from_numpy(positions).cuda()
    _, kp = h3.qk_norm_rope(None, to_device(k), None, None if wk is None else to_device(wk),
                            rope=rope, rope_theta=1e6, positions=pos_dev)
    o, lse = h3.gqa_causal_qnorm_rope_fwd(to_device(q), kp, to_device(v),
                                          q_norm_weight=None if wq is None else to_device(wq),
                                          rope=rope, rope_theta=1e6, positions=pos_dev,
                                          softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse, kp


CASES = [  # S, Hq, Hkv, D, seed, norm, rope, explicit positions
    (1, 8, 1, 128, 701, True, True, False),
    (97, 16, 2, 128, 702, True, True, False),    # G = 8, ragged
    (300, 64, 8, 128, 703, True, True, False),   # the encoder's heads
    (129, 16, 4, 128, 704, True, True, True),    # G = 4, positions given
    (200, 8, 4, 128, 705, False, True, False),   # G = 2, RoPE only
    (64, 4, 4, 64, 706, True, False, False),     # D = 64 MHA, norm only
    (333, 8, 2, 64, 707, True, True, True),      # D = 64, G = 4
    (260, 16, 2, 64, 708, True, True, False),    # D = 64, G = 8
    (150, 16, 2, 128, 709, True, True, "far"),   # positions near 10^5 (fp64 angle reduction)
    (517, 4, 4, 64, 710, True, True, False),     # D = 64, G = 1, several blocks, ragged
    (190, 8, 4, 64, 711, True, True, True),      # D = 64, G = 2
    (270, 8, 4, 128, 712, True, True, False),    # D = 128, G = 2, norm + RoPE
]


@pytest.mark.parametrize("S,Hq,Hkv,D,seed,norm,rope,explicit", CASES)
def test_qpro_small(lib, S, Hq, Hkv, D, seed, norm, rope, explicit):
    q, k, v = normal_inputs(seed, S, Hq, Hkv, D)
    wq = _weights(seed + 1000, D) if norm else None
    wk = _weights(seed + 2000, D) if norm else None
    positions = None
    if explicit == "far":
        positions = (100000 - np.arange(S, dtype=np.int32) * 7).astype(np.int32)
    elif explicit:
        positions = (np.arange(S, dtype=np.int32) * 3 + 5000).astype(np.int32)
    scale = workloads.default_scale(D)
    o, lse, kp = _run(lib, q, k, v, wq, wk, rope, positions, scale)
    rq = _prologue_ref(q, wq, rope, positions)
    rk = _prologue_ref(k, wk, rope, positions)
    o_ref, lse_ref = oracle.gqa_causal(rq, rk, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, f"qpro S={S} {Hq}/{Hkv} D={D}")


def test_k_only_prologue_matches_the_full_call(lib):
    """The K-only prologue (Hq = 0) writes exactly the K the two-tensor call writes."""
    import torch

    S, Hq, Hkv, D = 333, 16, 4, 128
    q, k, _ = normal_inputs(720, S, Hq, Hkv, D)
    wq, wk = _weights(721, D), _weights(722, D)
    _, k_both = lib.qk_norm_rope(to_device(q), to_device(k), to_device(wq), to_device(wk))
    q_none, k_only = lib.qk_norm_rope(None, to_device(k), None, to_device(wk))
    torch.cuda.synchronize()
    assert q_none is None
    assert np.array_equal(bits_of(k_only), bits_of(k_both))


def test_qpro_matches_the_two_pass_path(lib):
    """Q prologue inside the attention kernel vs the prologue kernel then the plain causal
    call: the same function, so the outputs agree to within the attention tolerance."""
    import torch

    S, Hq, Hkv, D = 1000, 64, 8, 128
    q, k, v = normal_inputs(730, S, Hq, Hkv, D)
    wq, wk = _weights(731, D), _weights(732, D)
    scale = workloads.default_scale(D)
    qp, kp = lib.qk_norm_rope(to_device(q), to_device(k), to_device(wq), to_device(wk))
    o2, lse2 = lib.gqa_causal_fwd(qp, kp, to_device(v), softmax_scale=scale)
    o1, lse1 = lib.gqa_causal_qnorm_rope_fwd(to_device(q), kp, to_device(v),
                                             q_norm_weight=to_device(wq), softmax_scale=scale)
    torch.cuda.synchronize()
    a1, a2 = to_f64(o1), to_f64(o2)
    rel = np.linalg.norm(a1 - a2) / np.linalg.norm(a2)
    print(f"[qpro] fused vs two-pass: rel_l2={rel:.3e} max_abs={np.abs(a1 - a2).max():.3e} "
          f"lse_abs={np.abs(to_f64(lse1) - to_f64(lse2)).max():.3e}", flush=True)
    assert rel <= 5e-3 and np.abs(a1 - a2).max() <= 2e-2
    assert np.abs(to_f64(lse1) - to_f64(lse2)).max() <= 1e-3


def test_qpro_primary_size_sampled(lib):
    """The primary workload (S=10231, 64/8 heads, D=128, ragged tail) with norm + RoPE, in
    the launch configuration of the benchmark, on sampled query tokens (every head)."""
    import torch

    w = workloads.WORKLOADS[workloads.PRIMARY]
    inp = workloads.generate(w)
    wq, wk = _weights(740, 128), _weights(741, 128)
    o, lse, _ = _run(lib, inp["q"], inp["k"], inp["v"], wq, wk, True, None, w.scale)
    rq = _prologue_ref(inp["q"], wq, True, None)
    rk = _prologue_ref(inp["k"], wk, True, None)
    tokens = workloads.sample_tokens(w.seqlens, 24, seed=742)
    o_ref, lse_ref = oracle.gqa_causal(rq, rk, inp["v"], w.scale, tokens=tokens)
    tok_t = torch.from_numpy(tokens).to("cuda")
    assert_close(to_f64(o.index_select(0, tok_t)), to_f64(lse.index_select(1, tok_t)), o_ref,
                 lse_ref, f"qpro primary ({len(tokens)} sampled tokens)")
