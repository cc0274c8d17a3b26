"""The fp64 oracle against brute force, a library routine, closed forms,
invariants and 50-digit results (CPU only)."""

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_arguments(orc):
    import numpy as np

    q = np.zeros((4, 4, 8), np.uint16)
    k = np.zeros((4, 3, 8), np.uint16)  # 4 query heads do not split into 3 groups
    with pytest.raises(ValueError):
        orc.gqa_causal(q, k, k, 1.0)
    k = np.zeros((4, 2, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.gqa_causal(q, k, k, 1.0, tokens=[4])  # past the end
    with pytest.raises(ValueError):
        orc.gqa_causal_varlen(q, k, k, [0, 3, 2, 4], 1.0)  # decreasing offsets


def test_thread_count_does_not_change_results(orc):
    import numpy as np
    from workloads import normal_inputs

    q, k, v = normal_inputs(60, 200, 8, 2, 32)
    o1, l1 = orc.gqa_causal(q, k, v, 0.2, threads=1)
    o4, l4 = orc.gqa_causal(q, k, v, 0.2, threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)
