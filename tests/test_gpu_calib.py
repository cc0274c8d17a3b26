"""The calibration loops behind the bench line's matrix-core and exponential ceilings,
through the C ABI entry h3attn_calib_loop (needs a gfx950 GPU): every wave records its
stamps, the counters move forward, and the cycles per instruction fall in the range the
instruction can take (a v_mfma_f32_32x32x16_bf16 occupies the matrix core for 32 cycles
at one wave per SIMD and 48 per wave at two; a v_exp_f32 of a whole wave takes a few to a
few tens of cycles).  The paired kind runs two workgroups per compute unit."""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h3():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import causal_grouped_query_amd as h3

    h3.load_library()
    return h3


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield


@pytest.mark.parametrize("kind,per_iter,lo,hi,wps", [(0, 8, 30.0, 80.0, 1), (2, 8, 30.0, 80.0, 1),
                                                     (1, 16, 2.0, 64.0, 1),
                                                     (3, 8, 30.0, 120.0, 2)])
def test_calib_loop_stamps(h3, kind, per_iter, lo, hi, wps):
    import torch

    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 256
    stamps, khz = h3.calib_loop(kind, wps * ncu, iters)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy()
    assert st.shape == (wps * ncu * 4, 4)
    assert khz > 0
    cycles, ticks = st[:, 1] - st[:, 0], st[:, 3] - st[:, 2]
    assert (cycles > 0).all() and (ticks > 0).all()          # every wave wrote its stamps
    per_instr = np.median(cycles) / (iters * per_iter)
    assert lo <= per_instr <= hi, per_instr
    ghz = np.median(cycles / (ticks / (khz * 1e3))) / 1e9
    assert 0.5 <= ghz <= 2.6, ghz                             # a shader clock, not a fixed one


def test_calib_loop_reuses_buffers(h3):
    import torch

    n = 8
    stamps = torch.zeros((n * 4, 4), dtype=torch.int64, device="cuda")
    sink = torch.full((n * 256,), float("nan"), dtype=torch.float32, device="cuda")
    out, _ = h3.calib_loop(h3.CALIB_EXP, n, 32, stamps=stamps, sink=sink)
    torch.cuda.synchronize()
    assert out.data_ptr() == stamps.data_ptr()
    assert torch.isfinite(sink).all()                         # every thread wrote its value
    with pytest.raises(ValueError):
        h3.calib_loop(h3.CALIB_EXP, n + 1, 32, stamps=stamps, sink=sink)
