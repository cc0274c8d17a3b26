"""The synthetic workloads use the sequence lengths the issue prints, and the
seeded generators are deterministic and round to bf16 correctly (CPU only)."""

import os

import numpy as np

import workloads
from workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "issue_sequence_lengths.txt")


def _golden():
    lengths, extra = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0].isdigit():
                lengths.append(int(parts[0]))
            else:
                extra[parts[0]] = int(parts[1])
    return lengths, extra


def test_failing_lengths_match_issue_table():
    lengths, extra = _golden()
    assert sorted(lengths) == sorted(workloads.FAILING_LENGTHS)
    w = WORKLOADS["varlen_4x_t35124"]
    assert sorted(w.seqlens) == sorted(lengths)
    assert list(w.cu_seqlens) == [0, 8184, 16383, 24893, 35124]
    assert WORKLOADS["failing_s10231"].seqlens == (10231,)
    # the under-cap workload sits below the ceiling the issue quotes
    assert WORKLOADS["under_cap_s7680"].seqlens[0] < extra["approx_ceiling"]
    assert extra["threadgroup_bytes"] // 4 < 10231


def test_flop_count_of_primary_workload():
    w = WORKLOADS["failing_s10231"]
    assert w.kept_pairs_per_head() == 10231 * 10232 // 2 == 52341796
    assert w.causal_flop() == 4 * 128 * 64 * 52341796


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 2**-7 + 2**-8, -3.0e-3, 65504.0, 1.0 + 2**-8 + 2**-20],
                 dtype=np.float32)
    b = workloads.f32_to_bf16_bits(x)
    back = workloads.bf16_bits_to_f32(b)
    # ties go to the even mantissa; above-tie rounds up
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2**-6
    assert back[5] == 1.0 + 2**-7
    rel = np.abs(back - x) / np.abs(x)
    assert np.all(rel <= 2.0**-8)  # unit roundoff of an 8-bit significand
    torch = __import__("torch")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_generators_are_seeded():
    a = workloads.normal_inputs(7, 33, 8, 2, 16)
    b = workloads.normal_inputs(7, 33, 8, 2, 16)
    c = workloads.normal_inputs(8, 33, 8, 2, 16)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])


def test_stress_generator_ties_spike_keys():
    q, k, v, pos = workloads.stress_inputs(5, 400, 8, 2, 16)
    assert len(pos) == 20
    assert np.all(k[pos] == k[pos[0]][None])
    vf = workloads.bf16_bits_to_f32(v)
    assert vf.min() >= -1.0 and vf.max() <= 1.0


def test_sample_tokens_cover_edges():
    t = workloads.sample_tokens((8184, 8199), 16, seed=3)
    for must in (0, 8183, 8184, 8184 + 8198, 63, 64):
        assert must in t
    assert t.max() < 8184 + 8199


def test_block_tokens_one_per_query_block_with_moving_offset():
    t = workloads.block_tokens([70, 5, 64])
    assert t.tolist() == [0, 33, 66, 70, 75, 108]
    # the S=10231 workload: 320 blocks of 32 tokens, offsets 0, 1, .., 31, 0, 1, ..
    t = workloads.block_tokens([10231])
    assert len(t) == 320
    assert all(int(x) // 32 == b and int(x) % 32 == b % 32 for b, x in enumerate(t[:-1]))
    assert int(t[-1]) == 10230
