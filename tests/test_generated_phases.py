"""The generated inner loop of the head-dim-128 kernel (CPU only): the committed
csrc/tile_phases.inc is what csrc/gen_tile_phases.py writes, and the generator's own
schedule checks hold (and reject a schedule known to be wrong)."""

import importlib.util
import os
import subprocess
import sys

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "causal_grouped_query_amd", "csrc")
GEN = os.path.join(CSRC, "gen_tile_phases.py")


def _generator():
    spec = importlib.util.spec_from_file_location("gen_tile_phases", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_committed_phases_match_the_generator():
    r = subprocess.run([sys.executable, GEN, "--check"], cwd=CSRC, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


def test_phase_counts():
    g = _generator()
    units, lines = g.phase_lines(128, True, True, True, g.FILLS_PER_PHASE, False)
    assert sum(ln.startswith("v_mfma") for ln in lines) == 32          # 16 score + 16 P.V
    assert sum(ln.startswith("v_exp_f32") for ln in lines) == 32       # one per score
    assert sum(ln.startswith("buffer_load_dwordx4") for ln in lines) == g.FILLS_PER_PHASE
    assert sum(ln.startswith("ds_read_b128") for ln in lines) == 8     # K fragments
    assert sum(ln.startswith("ds_read_b64_tr_b16") for ln in lines) == 16


def test_reading_three_units_ahead_is_rejected():
    """With LDS reads three fragment units ahead a read refills the buffer of the MFMA just
    issued before it; the GPU gave wrong results for that schedule."""
    g = _generator()
    g.AHEAD = 3
    up = g.phase_lines(128, True, True, True, g.FILLS_PER_PHASE, False)[1]
    down = g.phase_lines(128, True, True, True, g.FILLS_PER_PHASE, True)[1]
    with pytest.raises(AssertionError):
        g.check_fragment_reuse(up + down)
