"""Causal GQA forward with the Q prologue (RMS norm + RoPE) inside the attention kernel,
h3attn_gqa_causal_qnorm_rope_fwd, against the fp64 oracle (needs a gfx950 GPU).

Reference: the oracle's prologue of Q and of K, each rounded to bf16 (the prologue's
output type), then the oracle's causal attention.  The GPU side transforms K with the
K-only prologue call and Q inside the attention kernel.

The prologue's output is rounded to bf16 once, from fp32 arithmetic on the GPU and from
fp64 in the oracle.  Where the exact value lies within the fp32 error of a midpoint between
two bf16 values both roundings are correct, and the GPU's Q or K element may be one bf16
step away from the oracle's.  O stays far inside its tolerances; LSE, which follows the
largest score of a row, gets for each row the bound such steps can move it by on top of
its usual 1e-3 (LSE is 1-Lipschitz in the max-norm of the scores; the bound is zero for
rows with no such element).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, bits_of, errors, to_device, to_f64
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, normal_inputs

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


# relative distance from a bf16 midpoint within which an fp32 evaluation of the prologue
# (a sum of D squares, a reciprocal square root, products with the weight, cos and sin)
# may land on either side of it: far above its relative error of a few times 2^-24
AMBIGUOUS_REL = 2.0 ** -18


def _prologue_ref(x, w, rope, positions):
    """The oracle's prologue rounded to bf16 (bits), and per element the bf16 step by which a
    correct fp32 evaluation may round the other way (0 where it cannot)."""
    exact = oracle.qk_norm_rope(x, weight=w, rope=rope, theta=1e6, positions=positions)
    bits = f32_to_bf16_bits(exact.astype(np.float32))
    a = np.abs(exact)
    lo_bits = (a.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    lo = bf16_bits_to_f32(lo_bits).astype(np.float64)
    hi = bf16_bits_to_f32(lo_bits + np.uint16(1)).astype(np.float64)
    step = np.where(np.abs(a - 0.5 * (lo + hi)) <= AMBIGUOUS_REL * a, hi - lo, 0.0)
    return bits, step


def _lse_budget(rq, q_step, rk, k_step, scale, tokens=None, k_steps_too=True):
    """[Hq, tokens] bound on the move of a row's LSE when the Q and K elements with a nonzero
    step are one bf16 step off.  A causal score s_ij = scale <q_i, k_j> (j <= i) then moves
    by |ds_ij| <= scale * (sum_d q_step[i,d] |k_jd| + sum_d |q_id| k_step[j,d]) (magnitudes
    taken after a step), and LSE_i moves by at most sum_j p_ij |ds_ij| + max_j |ds_ij|^2 / 2
    (its gradient is the row's softmax p_i, its curvature at most 1/2), p_i from the
    reference's own scores."""
    Hq, Hkv = rq.shape[1], rk.shape[1]
    G = Hq // Hkv
    sel = np.arange(rq.shape[0]) if tokens is None else np.asarray(tokens)
    later = np.arange(rk.shape[0])[None, None, :] > sel[:, None, None]   # keys past the row
    qv = bf16_bits_to_f32(rq[sel]).astype(np.float64)                  # [n, Hq, D]
    qa = np.abs(qv) + q_step[sel]
    out = np.zeros((len(sel), Hq))
    for kv in range(Hkv):
        hs = slice(kv * G, (kv + 1) * G)
        kvals = bf16_bits_to_f32(rk[:, kv, :]).astype(np.float64)         # [S, D]
        ka = np.abs(kvals) + k_step[:, kv, :]
        n = len(sel)

        def rows_by_keys(a, b):   # [n, G, D] x [S, D] -> [n, G, S]
            return (np.ascontiguousarray(a).reshape(n * G, -1) @ b.T).reshape(n, G, -1)

        sc = scale * rows_by_keys(qv[:, hs, :], kvals)
        sc[np.broadcast_to(later, sc.shape)] = -np.inf
        p = np.exp(sc - sc.max(axis=2, keepdims=True))
        p /= p.sum(axis=2, keepdims=True)
        ds = rows_by_keys(q_step[sel][:, hs, :], ka)                           # Q steps
        if k_steps_too:
            ds += rows_by_keys(qa[:, hs, :], np.ascontiguousarray(k_step[:, kv, :]))  # K steps
        ds *= scale
        ds[np.broadcast_to(later, ds.shape)] = 0.0
        out[:, hs] = (p * ds).sum(axis=2) + 0.5 * ds.max(axis=2) ** 2
    return out.T


def _assert_close(o, lse, o_ref, lse_ref, budget, what):
    og, lg = to_f64(o), to_f64(lse)
    rel, mx, lmx = errors(og, lg, o_ref, lse_ref)
    over = float((np.abs(lg - lse_ref) - budget).max())
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs={mx:.3e} lse_abs={lmx:.3e} "
          f"(beyond the rows' rounding bounds {over:.3e}; largest bound {budget.max():.3e})",
          flush=True)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), f"{what}: non-finite"
    assert rel <= O_REL_L2, f"{what}: O relative L2 {rel:.3e}"
    assert mx <= O_MAX_ABS, f"{what}: O max abs {mx:.3e}"
    assert over <= LSE_MAX_ABS, f"{what}: LSE {over:.3e} beyond its bound"


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
    rq, q_step = _prologue_ref(q, wq, rope, positions)
    rk, k_step = _prologue_ref(k, wk, rope, positions)
    o_ref, lse_ref = oracle.gqa_causal(rq, rk, v, scale)
    _assert_close(o, lse, o_ref, lse_ref, _lse_budget(rq, q_step, rk, k_step, scale),
                  f"qpro S={S} {Hq}/{Hkv} D={D}")


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
    # both paths use the same K; their Q may differ by one step where either rounding is
    # correct
    rq, q_step = _prologue_ref(q, wq, True, None)
    rk, k_step = _prologue_ref(k, wk, True, None)
    budget = _lse_budget(rq, q_step, rk, k_step, scale, k_steps_too=False)
    _assert_close(o1, lse1, to_f64(o2), to_f64(lse2), budget, "qpro fused vs two-pass")


def test_qpro_primary_size_sampled(lib):
    """The primary workload (S=10231, 64/8 heads, D=128, ragged tail) with norm + RoPE, in
    the launch configuration of the benchmark, on sampled query tokens (every head)."""
    import torch

    w = workloads.WORKLOADS[workloads.PRIMARY]
    inp = workloads.generate(w)
    wq, wk = _weights(740, 128), _weights(741, 128)
    o, lse, _ = _run(lib, inp["q"], inp["k"], inp["v"], wq, wk, True, None, w.scale)
    rq, q_step = _prologue_ref(inp["q"], wq, True, None)
    rk, k_step = _prologue_ref(inp["k"], wk, True, None)
    tokens = workloads.sample_tokens(w.seqlens, 24, seed=742)
    o_ref, lse_ref = oracle.gqa_causal(rq, rk, inp["v"], w.scale, tokens=tokens)
    tok_t = torch.from_numpy(tokens).to("cuda")
    _assert_close(o.index_select(0, tok_t), lse.index_select(1, tok_t), o_ref, lse_ref,
                  _lse_budget(rq, q_step, rk, k_step, w.scale, tokens=tokens),
                  f"qpro primary ({len(tokens)} sampled tokens)")
