"""HIP path against the fp64 oracle, through the C ABI (needs a gfx950 GPU).

Small shapes are compared element by element over every output; the five
named workloads run at full size in the same launch configuration the
benchmark times and are compared on sampled query tokens (every head), plus
properties that hold at any size.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, bits_of, to_device, to_f64
from workloads import WORKLOADS, normal_inputs, stress_inputs

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


def _run(h3, q, k, v, scale):
    import torch

    o, lse = h3.gqa_causal_fwd(to_device(q), to_device(k), to_device(v), softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


# (S, Hq, Hkv, D, seed): every group size and head dim, lengths around tile edges
SMALL = [
    (256, 8, 2, 64, 1),      # the tiny workload
    (1, 8, 8, 128, 101),
    (2, 8, 1, 128, 102),
    (31, 16, 4, 128, 103),
    (63, 16, 2, 128, 104),
    (64, 8, 8, 64, 105),
    (65, 4, 4, 64, 106),
    (129, 16, 8, 64, 107),
    (200, 16, 2, 128, 108),
    (333, 64, 8, 128, 109),
    (517, 8, 4, 64, 110),
    (700, 8, 8, 128, 111),
    (1000, 16, 16, 128, 112),
    (97, 16, 2, 64, 113),      # G = 8 at D = 64
    (300, 32, 4, 64, 114),     # G = 8 at D = 64, several query blocks
    (130, 32, 8, 64, 115),     # G = 4 at D = 64
    (96, 64, 8, 128, 116),     # the 64/8/128 heads, exactly three 32-token query blocks
    (1025, 64, 8, 128, 117),   # the 64/8/128 heads, one token past a 1024 boundary
]


@pytest.mark.parametrize("S,Hq,Hkv,D,seed", SMALL)
def test_small_full_parity(lib, S, Hq, Hkv, D, seed):
    q, k, v = normal_inputs(seed, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    o, lse = _run(lib, q, k, v, scale)
    o_ref, lse_ref = oracle.gqa_causal(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, f"S={S} Hq={Hq} Hkv={Hkv} D={D}")


def test_large_logits_small(lib):
    """Logits with sigma ~ 16 (Q, K ~ 4 N(0,1)) and tied spike keys, small S."""
    q, k, v, _ = stress_inputs(120, 777, 16, 2, 128)
    scale = workloads.default_scale(128)
    o, lse = _run(lib, q, k, v, scale)
    o_ref, lse_ref = oracle.gqa_causal(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, "stress S=777")


def _jump_and_ramp_inputs(S):
    """Hq = 8 query heads on one KV head, D = 128, scores built on two key coordinates: key
    150's first coordinate is 128 (every other key's is 0) and the second coordinate ramps
    as j / 4.  Head 0 (q = 16 e0) meets a score ~181 above all earlier ones at key 150, so
    its weights overflow against any running max set before it; head 1 (q = -16 e0) sees
    that key ~181 below the rest; head 2 (q = 0) weights every key equally; head 3
    (q = 16 e1) has a max that grows by ~0.35 per key, ~106 over the row; heads 4-7 mix
    the two.  V is N(0,1)/2."""
    rng = np.random.Generator(np.random.PCG64(131))
    D = 128
    q = np.zeros((S, 8, D), np.float32)
    k = np.zeros((S, 1, D), np.float32)
    k[150 % S, 0, 0] = 128.0
    k[:, 0, 1] = np.arange(S, dtype=np.float32) / 4.0
    k[:, 0, 2:] = rng.standard_normal((S, D - 2), dtype=np.float32) * 0.5
    q[:, 0, 0], q[:, 1, 0], q[:, 3, 1] = 16.0, -16.0, 16.0
    q[:, 4, 0], q[:, 4, 1] = 8.0, 8.0
    q[:, 5, 0], q[:, 5, 1] = -8.0, 12.0
    q[:, 6, 2:] = rng.standard_normal((S, D - 2), dtype=np.float32)
    q[:, 7, 0], q[:, 7, 2:] = 4.0, rng.standard_normal((S, D - 2), dtype=np.float32)
    # rows led by one key return about that key's value row: V at half scale keeps |O|
    # under ~2, where the absolute O bound applies (a bf16 step there is 2^-7)
    v = rng.standard_normal((S, 1, D), dtype=np.float32) * 0.5
    return tuple(workloads.f32_to_bf16_bits(x) for x in (q, k, v))


@pytest.mark.parametrize("S", [300, 777])
def test_score_jumps_and_ramps(lib, S):
    """Scores that jump far above the running max (weights overflow to infinity and the
    row takes the max path), far below it (underflow), or grow steadily over the row
    (repeated raises), causal and bidirectional, against the oracle."""
    q, k, v = _jump_and_ramp_inputs(S)
    scale = workloads.default_scale(128)
    o, lse = _run(lib, q, k, v, scale)
    o_ref, lse_ref = oracle.gqa_causal(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, f"jumps and ramps S={S} causal")
    ob, lb = lib.gqa_fwd(to_device(q), to_device(k), to_device(v), causal=False,
                         softmax_scale=scale)
    ob_ref, lb_ref = oracle.gqa_bidirectional(q, k, v, scale)
    assert_close(to_f64(ob), to_f64(lb), ob_ref, lb_ref, f"jumps and ramps S={S} bidirectional")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_sampled(lib, name):
    """Full-size workload on the GPU; oracle on sampled query tokens (all heads)."""
    import torch

    w = WORKLOADS[name]
    inp = workloads.generate(w)
    q, k, v = to_device(inp["q"]), to_device(inp["k"]), to_device(inp["v"])
    if w.varlen:
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
        o, lse = lib.gqa_causal_varlen_fwd(q, k, v, cu, max(w.seqlens), softmax_scale=w.scale)
    else:
        o, lse = lib.gqa_causal_fwd(q, k, v, softmax_scale=w.scale)
    torch.cuda.synchronize()
    n_random = 24 if w.total_tokens > 20000 else 48
    tokens = workloads.sample_tokens(w.seqlens, n_random, seed=w.seed + 1000)
    if w.total_tokens <= 4096:
        tokens = np.arange(w.total_tokens)
    o_ref, lse_ref = oracle.gqa_causal_varlen(inp["q"], inp["k"], inp["v"], w.cu_seqlens, w.scale,
                                              tokens=tokens)
    tok_t = torch.from_numpy(tokens).to("cuda")
    o_s = to_f64(o.index_select(0, tok_t))
    lse_s = to_f64(lse.index_select(1, tok_t))
    assert_close(o_s, lse_s, o_ref, lse_ref, f"{name} ({len(tokens)} sampled tokens)")

    # properties over every output: finite, and each O row is a convex combination of
    # value rows, so |O[., h, d]| <= max_j |V[j, g, d]| (plus bf16 rounding)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    vmax = v.float().abs().amax(dim=0)                                  # [Hkv, D]
    bound = vmax.repeat_interleave(w.group, dim=0) * (1 + 2**-7) + 1e-6  # [Hq, D]
    assert bool((o.float().abs().amax(dim=0) <= bound).all())


def test_row_zero_is_v0_and_zero_query_prefix_mean(lib):
    import torch

    S, Hq, Hkv, D = 300, 16, 2, 128
    q, k, v = normal_inputs(130, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    o, lse = _run(lib, q, k, v, scale)
    ob = bits_of(o)
    G = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(ob[0, h], v[0, h // G]), f"row 0 of head {h} is not V[0]"
    # Q = 0: every visible score is zero -> prefix mean, LSE = ln(i+1)
    qz = np.zeros_like(q)
    o, lse = _run(lib, qz, k, v, scale)
    o_ref, lse_ref = oracle.gqa_causal(qz, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, "Q=0")
    np.testing.assert_allclose(to_f64(lse), np.log(np.arange(1, S + 1))[None].repeat(Hq, 0),
                               atol=1e-3, rtol=0)
    torch.cuda.synchronize()


def test_causality_bit_identical(lib):
    """Changing tokens >= t leaves rows < t bit-identical (masked weights are exactly 0)."""
    S, Hq, Hkv, D = 450, 16, 2, 128
    q, k, v = normal_inputs(131, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    o1, l1 = _run(lib, q, k, v, scale)
    b1, lb1 = bits_of(o1), to_f64(l1)
    for t in (1, 100, 257, 449):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[t:], k2[t:], v2[t:] = normal_inputs(132 + t, S - t, Hq, Hkv, D, sigma=3.0)
        o2, l2 = _run(lib, q2, k2, v2, scale)
        assert np.array_equal(b1[:t], bits_of(o2)[:t]), f"rows < {t} changed"
        assert np.array_equal(lb1[:, :t], to_f64(l2)[:, :t]), f"LSE rows < {t} changed"


@pytest.mark.parametrize("Hq,Hkv,D,seed", [
    (16, 2, 128, 140),   # G = 8
    (8, 4, 128, 141),    # G = 2
    (8, 8, 64, 142),     # G = 1
    (16, 4, 64, 143),    # G = 4
    (8, 1, 64, 144),     # G = 8
])
def test_varlen_equals_single_calls(lib, Hq, Hkv, D, seed):
    """A packed batch gives bit-identical results to one call per sequence,
    including empty sequences and lengths that are not multiples of any tile,
    for the packed instance of each group size and head dim checked."""
    import torch

    lens = [130, 0, 1, 64, 517, 0, 33]
    T = sum(lens)
    q, k, v = normal_inputs(seed, T, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, lse = lib.gqa_causal_varlen_fwd(qd, kd, vd, torch.from_numpy(cu).cuda(), max(lens),
                                       softmax_scale=scale)
    torch.cuda.synchronize()
    ob, lf = bits_of(o), to_f64(lse)
    for s, n in enumerate(lens):
        if n == 0:
            continue
        a, b = cu[s], cu[s + 1]
        o1, l1 = _run(lib, q[a:b], k[a:b], v[a:b], scale)
        assert np.array_equal(ob[a:b], bits_of(o1)), f"sequence {s} differs"
        assert np.array_equal(lf[:, a:b], to_f64(l1)), f"sequence {s} LSE differs"
    o_ref, lse_ref = oracle.gqa_causal_varlen(q, k, v, cu, scale)
    assert_close(to_f64(o), lf, o_ref, lse_ref, f"varlen mixed lengths {Hq}/{Hkv} D={D}")


def test_varlen_offsets_check_under_env_switch(lib, monkeypatch):
    """With H3ATTN_CHECK_CU_SEQLENS=1 the packed call reads the offsets back and refuses a
    max_seqlen below the longest sequence (and a malformed table) before launching; with
    valid arguments it gives the same bits as the unchecked call."""
    import torch

    lens = [40, 130, 7]
    T = sum(lens)
    q, k, v = normal_inputs(150, T, 16, 2, 128)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    monkeypatch.setenv("H3ATTN_CHECK_CU_SEQLENS", "1")
    sentinel = torch.full((T, 16, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o = sentinel.clone()
    for bad_cu, max_seqlen in ((cu, 129), (cu, 1), (torch.tensor([0, 40, 30, T], dtype=torch.int32,
                                                                  device="cuda"), 130)):
        with pytest.raises(lib.H3AttnError) as err:
            lib.gqa_causal_varlen_fwd(qd, kd, vd, bad_cu, max_seqlen, out=o)
        assert err.value.status == lib.ERR_SHAPE
        torch.cuda.synchronize()
        assert torch.equal(o, sentinel), "a refused call wrote its output"
    o1, l1 = lib.gqa_causal_varlen_fwd(qd, kd, vd, cu, 130)
    monkeypatch.delenv("H3ATTN_CHECK_CU_SEQLENS")
    o2, l2 = lib.gqa_causal_varlen_fwd(qd, kd, vd, cu, 130)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # host offsets: checked by the binding, then copied to the device
    o3, l3 = lib.gqa_causal_varlen_fwd(qd, kd, vd, cu.cpu(), 130)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    with pytest.raises(lib.H3AttnError) as err:
        lib.gqa_causal_varlen_fwd(qd, kd, vd, cu.cpu(), 129, out=o)
    assert err.value.status == lib.ERR_SHAPE


def test_deterministic_and_lse_optional(lib):
    import torch

    S, Hq, Hkv, D = 600, 64, 8, 128
    q, k, v = normal_inputs(150, S, Hq, Hkv, D)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o1, l1 = lib.gqa_causal_fwd(qd, kd, vd)
    o2, l2 = lib.gqa_causal_fwd(qd, kd, vd)
    o3, l3 = lib.gqa_causal_fwd(qd, kd, vd, return_lse=False)
    torch.cuda.synchronize()
    assert l3 is None
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, o3)


def test_outputs_stay_in_bounds(lib):
    """Guard regions around O and LSE (filled with NaN) are left untouched."""
    import torch

    S, Hq, Hkv, D = 211, 16, 4, 64
    q, k, v = normal_inputs(160, S, Hq, Hkv, D)
    guard = 4096
    n_o, n_l = S * Hq * D, Hq * S
    obuf = torch.full((n_o + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((n_l + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[guard:guard + n_o].view(S, Hq, D)
    lse = lbuf[guard:guard + n_l].view(Hq, S)
    lib.gqa_causal_fwd(to_device(q), to_device(k), to_device(v), out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isnan(obuf[:guard].float()).all() and torch.isnan(obuf[-guard:].float()).all())
    assert bool(torch.isnan(lbuf[:guard]).all() and torch.isnan(lbuf[-guard:]).all())
    assert bool(torch.isfinite(o.float()).all() and torch.isfinite(lse).all())


def test_empty_inputs_are_noops(lib):
    import torch

    z = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = lib.gqa_causal_fwd(z, zk, zk)
    assert o.shape == (0, 8, 128) and lse.shape == (8, 0)
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, lse = lib.gqa_causal_varlen_fwd(z, zk, zk, cu, 0)
    torch.cuda.synchronize()


def test_rejects_bad_arguments_on_gpu(lib):
    import torch

    q = torch.zeros((8, 8, 96), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((8, 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.H3AttnError) as e:
        lib.gqa_causal_fwd(q, k, k)
    assert e.value.status == lib.ERR_UNSUPPORTED
    q = torch.zeros((8, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((8, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.H3AttnError) as e:
        lib.gqa_causal_fwd(q, k, k, softmax_scale=float("nan"))
    assert e.value.status == lib.ERR_SCALE


# lengths around every boundary of the head-dim-128 kernel: 32-key sub-tiles, 64-key tiles,
# a wave's 64/G tokens, a workgroup's 256/G tokens, and the 4-stage ring wrapping
SWEEP_LENGTHS = sorted(set(list(range(1, 70)) + [95, 96, 97, 127, 128, 129, 191, 192, 193,
                                                 255, 256, 257, 287, 288, 289, 511, 512, 513]))


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (8, 8), (8, 4), (16, 4)])
def test_head_dim_128_length_sweep(lib, Hq, Hkv):
    """Every length in SWEEP_LENGTHS, causal and bidirectional, against the oracle: covers
    waves whose rows end before the workgroup's last sub-tile (fill-only phases), ragged
    last tiles and ring wrap-around for each group size."""
    import torch

    D = 128
    scale = workloads.default_scale(D)
    worst = (0.0, 0.0, 0.0)
    for S in SWEEP_LENGTHS:
        q, k, v = normal_inputs(1000 + S, S, Hq, Hkv, D)
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
        o, lse = lib.gqa_causal_fwd(qd, kd, vd, softmax_scale=scale)
        ob, lb = lib.gqa_fwd(qd, kd, vd, causal=False, softmax_scale=scale)
        torch.cuda.synchronize()
        for (og, lg), ref, what in (((o, lse), oracle.gqa_causal(q, k, v, scale), "causal"),
                                    ((ob, lb), oracle.gqa_bidirectional(q, k, v, scale),
                                     "bidirectional")):
            rel, mx, lmx = assert_close(to_f64(og), to_f64(lg), ref[0], ref[1],
                                        f"S={S} {Hq}/{Hkv} {what}")
            worst = tuple(max(a, b) for a, b in zip(worst, (rel, mx, lmx)))
    print(f"[parity] sweep {Hq}/{Hkv}: worst rel_l2={worst[0]:.3e} max_abs={worst[1]:.3e} "
          f"lse_abs={worst[2]:.3e}", flush=True)
