"""Split-KV (two-dispatch) path against the fp64 oracle, through the C ABI (needs a
gfx950 GPU).

The final O / LSE are compared with the full causal oracle; the per-split partials
left in the workspace are compared with the oracle's attention over each split's key
range (the ranges follow the published split rule), so the intermediate results are
pinned too, not only their merge.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, assert_close, to_device, to_f64
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


def _split(h3, q, k, v, scale, ns, workspace=None):
    import torch

    o, lse = h3.gqa_causal_splitkv_fwd(to_device(q), to_device(k), to_device(v), ns,
                                       softmax_scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def _tok_wg(G):
    return 256 // G


def _split_ranges(S, G, ns, block):
    """Key ranges [a, b) of every split of query block `block` (tiles of 64 keys)."""
    tok = _tok_wg(G)
    q0 = block * tok
    n = (min(q0 + tok, S) + 63) // 64
    first = [n * c // ns for c in range(ns + 1)]
    return [(64 * first[c], 64 * first[c + 1]) for c in range(ns)]


SMALL = [  # S, Hq, Hkv, D, seed, num_splits
    (256, 8, 2, 64, 1, 2),
    (1, 8, 8, 128, 201, 4),
    (65, 16, 2, 128, 202, 3),
    (300, 16, 4, 128, 203, 5),
    (333, 64, 8, 128, 204, 7),
    (517, 8, 8, 64, 205, 1),
    (700, 16, 16, 128, 206, 64),   # more splits than tiles: most are empty
    (1000, 8, 1, 64, 207, 4),
]


@pytest.mark.parametrize("S,Hq,Hkv,D,seed,ns", SMALL)
def test_splitkv_small_full_parity(lib, S, Hq, Hkv, D, seed, ns):
    q, k, v = normal_inputs(seed, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    o, lse = _split(lib, q, k, v, scale, ns)
    o_ref, lse_ref = oracle.gqa_causal(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref,
                 f"split-KV S={S} Hq={Hq} Hkv={Hkv} D={D} splits={ns}")


def test_splitkv_large_logits(lib):
    q, k, v, _ = stress_inputs(220, 777, 16, 2, 128)
    scale = workloads.default_scale(128)
    o, lse = _split(lib, q, k, v, scale, 3)
    o_ref, lse_ref = oracle.gqa_causal(q, k, v, scale)
    assert_close(to_f64(o), to_f64(lse), o_ref, lse_ref, "split-KV stress S=777")


@pytest.mark.parametrize("S,Hq,Hkv,D,ns", [(300, 8, 2, 128, 3), (600, 8, 8, 64, 4),
                                            (300, 16, 2, 128, 3), (200, 8, 1, 128, 5)])
def test_splitkv_partials_match_oracle_key_ranges(lib, S, Hq, Hkv, D, ns):
    """Each split's partial O and LSE in the workspace equal the oracle's attention over
    that split's key range; rows with no key in the range hold LSE = -inf."""
    import torch

    q, k, v = normal_inputs(230 + ns, S, Hq, Hkv, D)
    scale = workloads.default_scale(D)
    need = lib.splitkv_workspace_bytes(S, Hq, D, ns)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _split(lib, q, k, v, scale, ns, workspace=ws)
    o_bytes = ns * S * Hq * D * 4
    lse_off = (o_bytes + 255) // 256 * 256
    o_part = ws[:o_bytes].view(torch.float32).view(ns, S, Hq, D).double().cpu().numpy()
    lse_part = ws[lse_off:lse_off + ns * Hq * S * 4].view(torch.float32).view(ns, Hq, S)
    lse_part = lse_part.double().cpu().numpy()
    G = Hq // Hkv
    tok = _tok_wg(G)
    checked = 0
    for block in range((S + tok - 1) // tok):
        tokens = np.arange(block * tok, min((block + 1) * tok, S))
        for c, (a, b) in enumerate(_split_ranges(S, G, ns, block)):
            if a == b:
                continue                      # an empty split writes nothing
            o_ref, l_ref = oracle.gqa_causal_keyrange(q, k, v, scale, a, b, tokens=tokens)
            o_gpu = o_part[c, tokens]
            l_gpu = lse_part[c][:, tokens]
            empty = ~np.isfinite(l_ref)
            assert np.array_equal(~np.isfinite(l_gpu), empty), (block, c)
            assert np.all(o_gpu[empty.T] == 0.0), (block, c)
            full = ~empty
            if full.any():
                assert np.max(np.abs(l_gpu[full] - l_ref[full])) <= LSE_MAX_ABS, (block, c)
                diff = np.abs(o_gpu - o_ref)
                assert diff.max() <= O_MAX_ABS, (block, c, diff.max())
            checked += 1
    assert checked > 0


def test_splitkv_leaves_workspace_tail_alone(lib):
    """The call writes only inside the documented workspace size."""
    import torch

    S, Hq, Hkv, D, ns = 200, 8, 2, 128, 3
    q, k, v = normal_inputs(240, S, Hq, Hkv, D)
    need = lib.splitkv_workspace_bytes(S, Hq, D, ns)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    _split(lib, q, k, v, workloads.default_scale(D), ns, workspace=ws)
    assert bool((ws[need:] == 0x5A).all())


def test_splitkv_primary_workload_sampled(lib):
    """The primary workload (S=10231, 64/8/128) with 4 splits: sampled rows against the
    oracle, and the whole output against the single-dispatch kernel."""
    import torch

    w = WORKLOADS[workloads.PRIMARY]
    inp = workloads.generate(w)
    q, k, v = (to_device(inp[n]) for n in ("q", "k", "v"))
    o, lse = lib.gqa_causal_splitkv_fwd(q, k, v, 4, softmax_scale=w.scale)
    o1, lse1 = lib.gqa_causal_fwd(q, k, v, softmax_scale=w.scale)
    torch.cuda.synchronize()
    tokens = workloads.sample_tokens(w.seqlens, 24, seed=w.seed + 500)
    o_ref, lse_ref = oracle.gqa_causal(inp["q"], inp["k"], inp["v"], w.scale, tokens=tokens)
    idx = torch.from_numpy(tokens).cuda()
    assert_close(to_f64(o.index_select(0, idx)), to_f64(lse.index_select(1, idx)), o_ref, lse_ref,
                 "split-KV primary workload (sampled)")
    d = (o.float() - o1.float()).abs()
    rel = float(torch.linalg.vector_norm(o.float() - o1.float()) / torch.linalg.vector_norm(o1.float()))
    print(f"[parity] split vs single dispatch: rel {rel:.2e} max {float(d.max()):.2e} "
          f"lse {float((lse - lse1).abs().max()):.2e}", flush=True)
    assert rel <= O_REL_L2 and float(d.max()) <= O_MAX_ABS
    assert float((lse - lse1).abs().max()) <= LSE_MAX_ABS
