"""Host-side logic of bench.py (no GPU): the one-GPU guard and the rule that the
recorded HBM traffic is reported only for the kernel source it was measured on."""

import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

CSRC = os.path.join("causal_grouped_query_amd", "csrc")
KERNEL = os.path.join(CSRC, "gqa_fwd_kernel.hpp")
BODY = os.path.join(CSRC, "gqa_fwd_body.inc")
TRAFFIC = os.path.join("profiles", "gqa_causal_fwd_s10231_hbm_traffic.txt")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _fake_tree(tmp_path, kernel_text: bytes, recorded_hash: str, nbytes: int = 123456):
    (tmp_path / CSRC).mkdir(parents=True)
    (tmp_path / KERNEL).write_bytes(kernel_text)
    (tmp_path / BODY).write_bytes(b"")
    (tmp_path / "profiles").mkdir()
    (tmp_path / TRAFFIC).write_text(
        "header line\n"
        f"traffic_bytes_per_launch: {nbytes} source_sha256: {recorded_hash}\n")


def test_recorded_traffic_needs_the_measured_source(tmp_path, monkeypatch):
    text = b"// kernel source as profiled\n"
    _fake_tree(tmp_path, text, hashlib.sha256(text).hexdigest())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic() == 123456
    # any edit of the kernel source withdraws the figure
    (tmp_path / KERNEL).write_bytes(text + b"// edited\n")
    assert bench.recorded_traffic() is None


def test_recorded_traffic_missing_or_malformed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / CSRC).mkdir(parents=True)
    (tmp_path / KERNEL).write_bytes(b"x")
    (tmp_path / BODY).write_bytes(b"y")
    assert bench.recorded_traffic() is None            # no record at all
    (tmp_path / "profiles").mkdir()
    (tmp_path / TRAFFIC).write_text("traffic_bytes_per_launch: 5\n")
    assert bench.recorded_traffic() is None            # no hash on the line


def test_committed_traffic_record_matches_committed_kernel():
    """The HBM traffic under profiles/ was taken on the kernel source in the tree, so the
    benchmark line reports it (a kernel change must come with a new counter run)."""
    hs = hashlib.sha256()
    for path in (KERNEL, BODY):
        with open(os.path.join(ROOT, path), "rb") as f:
            hs.update(f.read())
    h = hs.hexdigest()
    with open(os.path.join(ROOT, TRAFFIC)) as f:
        lines = [ln.split() for ln in f if ln.startswith("traffic_bytes_per_launch:")]
    assert lines, "no traffic record in the profile"
    assert lines[-1][3] == h
    assert bench.recorded_traffic() == int(lines[-1][1])
    # well above the 379.7 MB the launch must move, well below a K/V re-read per block
    assert 3.8e8 <= bench.recorded_traffic() <= 2.0e9


def test_default_workload_is_the_metric_workload():
    import workloads

    w = workloads.ALL_WORKLOADS[workloads.PRIMARY]
    assert "S=10231" in bench.METRIC
    assert tuple(w.seqlens) == (10231,) and w.causal
    assert (w.n_q_heads, w.n_kv_heads, w.head_dim) == (64, 8, 128)
