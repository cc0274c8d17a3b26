"""Host-side logic of bench.py (no GPU): the one-GPU guard, the rule that figures recorded
from counter runs (HBM traffic, shader clock) are reported only for the kernel source they
were measured on, and the clock sampler's behaviour without a GPU."""

import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

CSRC = os.path.join("causal_grouped_query_amd", "csrc")
SOURCES = [os.path.join(CSRC, n) for n in bench.KERNEL_SOURCES]
TRAFFIC = bench.PROFILE
KEY = "traffic_bytes_per_launch"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _hash(texts):
    h = hashlib.sha256()
    for t in texts:
        h.update(t)
    return h.hexdigest()


def _fake_tree(tmp_path, texts, recorded_hash: str, nbytes: int = 123456):
    (tmp_path / CSRC).mkdir(parents=True)
    for path, t in zip(SOURCES, texts):
        (tmp_path / path).write_bytes(t)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / TRAFFIC).write_text(
        "header line\n"
        f"{KEY}: {nbytes} source_sha256: {recorded_hash}\n")


def test_recorded_figure_needs_the_measured_source(tmp_path, monkeypatch):
    texts = [f"// source file {i} as profiled\n".encode() for i in range(len(SOURCES))]
    _fake_tree(tmp_path, texts, _hash(texts))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded(TRAFFIC, KEY) == 123456
    # an edit of any of the sources withdraws the figure
    for path, t in zip(SOURCES, texts):
        (tmp_path / path).write_bytes(t + b"// edited\n")
        assert bench.recorded(TRAFFIC, KEY) is None
        (tmp_path / path).write_bytes(t)
    assert bench.recorded(TRAFFIC, KEY) == 123456
    assert bench.recorded(TRAFFIC, "no_such_key") is None      # another key is not there


def test_recorded_figure_missing_or_malformed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / CSRC).mkdir(parents=True)
    for path in SOURCES:
        (tmp_path / path).write_bytes(b"x")
    assert bench.recorded(TRAFFIC, KEY) is None            # no record at all
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / TRAFFIC).write_text(f"{KEY}: 5\n")
    assert bench.recorded(TRAFFIC, KEY) is None            # no hash on the line


def test_committed_records_match_committed_kernel():
    """The HBM traffic and the counter clock under profiles/ were taken on the kernel source
    in the tree, so the benchmark line reports them (a kernel change must come with new
    counter runs)."""
    h = bench.kernel_source_hash()
    for profile, key in ((TRAFFIC, KEY), (TRAFFIC, "clock_ghz")):
        with open(os.path.join(ROOT, "profiles", profile)) as f:
            lines = [ln.split() for ln in f if ln.startswith(key + ":")]
        assert lines, f"no {key} record in {profile}"
        assert lines[-1][3] == h, profile
        assert bench.recorded(profile, key) == float(lines[-1][1])
    # well above the 379.7 MB the launch must move, well below a K/V re-read per block
    assert 3.8e8 <= bench.recorded(TRAFFIC, KEY) <= 2.0e9
    assert 0.5 <= bench.recorded(TRAFFIC, "clock_ghz") <= 2.5


def test_clock_sampler_never_raises_without_a_gpu():
    s = bench.ClockSampler(period_s=0.001)
    s.start()
    s.stop()
    out = s.summary()
    assert "source" in out and "mhz_mean" in out
    if out["mhz_mean"] is None:
        assert out["error"]


def test_clock_sampler_keeps_each_refresh_inside_the_timed_region_once():
    s = bench.ClockSampler.__new__(bench.ClockSampler)
    s.error, s.period, s.window_begin = None, 0.005, None
    # (time, table counter, mean clock, XCD clocks, power): the table refreshes at t=0.5
    # (before the timed region), t=1.5 and t=2.5; the region is [1.0, 3.0]
    s.samples = [(0.1, 10, 400.0, [400] * 8, 250), (0.6, 11, 1900.0, [1900] * 8, 1300),
                 (1.2, 11, 1900.0, [1900] * 8, 1300), (1.6, 12, 2000.0, [2000] * 8, 1350),
                 (1.7, 12, 2000.0, [2000] * 8, 1350), (2.6, 13, 1800.0, [1800] * 8, 1360),
                 (3.2, 14, 500.0, [500] * 8, 300)]
    s.begin, s.end = 1.0, 3.0
    out = s.summary()
    assert out["refreshes"] == 2
    assert out["mhz_mean"] == 1900.0 and out["socket_power_w_mean"] == 1355.0
    s.begin, s.end = 1.0, 1.4           # no refresh inside: nothing is reported
    assert s.summary()["mhz_mean"] is None
    s.window_begin = 0.3                # a window opened before the timed region
    assert s.summary()["refreshes"] == 1 and s.summary()["mhz_mean"] == 1900.0


def test_default_workload_is_the_metric_workload():
    import workloads

    w = workloads.ALL_WORKLOADS[workloads.PRIMARY]
    assert "S=10231" in bench.METRIC
    assert tuple(w.seqlens) == (10231,) and w.causal
    assert (w.n_q_heads, w.n_kv_heads, w.head_dim) == (64, 8, 128)
