"""The largest token count the boundary accepts for 64 query / 8 KV heads at D = 128
(tokens * Hq * D = 2^31 - 8192, one token short of the 2^31 element limit), through the C
ABI, against the fp64 oracle on the rows with the highest indices (needs a gfx950 GPU).

The inputs (about 6 GB) are drawn on the GPU with torch's seeded generator; the oracle gets
the same bf16 values copied back.  Checked: one packed batch of 256 short sequences (first,
middle and last sequence in full), one 262143-token sequence (sampled rows, token-major and
head-major O), and the Q/K prologue over the same tensors (sampled rows).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, bits_of, to_f64

pytestmark = pytest.mark.gpu

HQ, HKV, D = 64, 8, 128
T_MAX = (2**31 - 1) // (HQ * D)          # 262143 tokens: T * Hq * D = 2^31 - 8192
assert T_MAX * HQ * D < 2**31 <= (T_MAX + 1) * HQ * D   # one more token is rejected (CPU test)


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


@pytest.fixture(scope="module")
def qkv():
    import torch

    q, k, v = workloads.device_normal_bf16(
        900, [(T_MAX, HQ, D), (T_MAX, HKV, D), (T_MAX, HKV, D)])
    torch.cuda.synchronize()
    yield q, k, v
    del q, k, v
    torch.cuda.empty_cache()


def test_varlen_at_index_limit(lib, qkv):
    import torch

    q, k, v = qkv
    lens = [1024] * 255 + [T_MAX - 255 * 1024]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert cu[-1] == T_MAX
    scale = workloads.default_scale(D)
    o, lse = lib.gqa_causal_varlen_fwd(q, k, v, torch.from_numpy(cu).cuda(), max_seqlen=1024,
                                       softmax_scale=scale)
    torch.cuda.synchronize()
    for s in (0, 128, 255):
        a, b = int(cu[s]), int(cu[s + 1])
        o_ref, lse_ref = oracle.gqa_causal(bits_of(q[a:b]), bits_of(k[a:b]), bits_of(v[a:b]),
                                           scale)
        assert_close(to_f64(o[a:b]), to_f64(lse[:, a:b]), o_ref, lse_ref,
                     f"varlen T={T_MAX} sequence {s} (tokens {a}..{b - 1})")


@pytest.mark.parametrize("head_major", [False, True])
def test_one_sequence_at_index_limit(lib, qkv, head_major):
    import torch

    q, k, v = qkv
    S = T_MAX
    scale = workloads.default_scale(D)
    o, lse = lib.gqa_fwd(q, k, v, causal=True, head_major_out=head_major, softmax_scale=scale)
    torch.cuda.synchronize()
    tokens = np.array([0, 1, 64, 12345, S // 2 + 7, S - 65, S - 2, S - 1], dtype=np.int64)
    idx = torch.from_numpy(tokens).cuda()
    # the oracle reads Q only at the sampled tokens: a zero array with those rows filled
    qh = np.zeros((S, HQ, D), dtype=np.uint16)
    qh[tokens] = bits_of(q.index_select(0, idx))
    o_ref, lse_ref = oracle.gqa_causal(qh, bits_of(k), bits_of(v), scale, tokens=tokens)
    o_s = (o.transpose(0, 1) if head_major else o).index_select(0, idx)
    assert_close(to_f64(o_s), to_f64(lse.index_select(1, idx)), o_ref, lse_ref,
                 f"S={S} sampled rows, head-major={head_major}")


def test_prologue_at_index_limit(lib, qkv):
    """Q/K RMS norm + RoPE over the same 262143-token tensors; sampled rows against the
    oracle with their token indices as positions."""
    import torch

    q, k, _ = qkv
    wq, wk = workloads.device_normal_bf16(901, [(D,), (D,)])
    qo, ko = lib.qk_norm_rope(q, k, wq, wk, eps=1e-6, rope=True, rope_theta=1e6)
    torch.cuda.synchronize()
    tokens = np.array([0, 777, T_MAX // 2, T_MAX - 2, T_MAX - 1], dtype=np.int64)
    idx = torch.from_numpy(tokens).cuda()
    for name, x, y, w in (("q", q, qo, wq), ("k", k, ko, wk)):
        ref = oracle.qk_norm_rope(bits_of(x.index_select(0, idx)), weight=bits_of(w), eps=1e-6,
                                  rope=True, theta=1e6, positions=tokens)
        got = workloads.bf16_bits_to_f32(bits_of(y.index_select(0, idx))).astype(np.float64)
        rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * rms
        worst = float((np.abs(got - ref) / np.maximum(bound, 1e-300)).max())
        print(f"[prologue] {name} at T={T_MAX}: worst err/bound {worst:.3f}", flush=True)
        assert np.all(np.abs(got - ref) <= bound), name
