"""The benchmark's host-side helpers (CPU): the committed profile summaries
parse, and what they hold is consistent with the algorithmic bytes."""
import os
import re

import bench

U = 22756352  # one fp32 encoder value map


def _text(path):
    assert os.path.exists(path), f"{path} is missing"
    return open(path).read()


def test_traffic_summary_parses_and_exceeds_the_algorithmic_bytes():
    text = _text(bench.TRAFFIC_FILE)
    assert re.search(r"kernel_source_sha256:\s*[0-9a-f]{16}", text)
    fwd = float(re.search(r"traffic_bytes_fwd:\s*([0-9.eE+]+)", text).group(1))
    bwd = float(re.search(r"traffic_bytes_bwd:\s*([0-9.eE+]+)", text).group(1))
    # HBM traffic can only exceed what the passes must move (3.5U and 6U)
    assert 3.5 * U <= fwd < 20 * U
    assert 6 * U <= bwd < 40 * U


def test_trace_summary_parses():
    text = _text(bench.TRACE_FILE)
    assert re.search(r"Kernel source sha256 \(first 16 hex\): `[0-9a-f]{16}`", text)
    fwd = float(re.search(r"Forward \(fwd_kernel\) average: ([0-9.]+) us", text).group(1))
    bwd = float(re.search(r"Backward \(sum of the averages of its \d+ kernels per call\): ([0-9.]+) us",
                          text).group(1))
    assert 0 < fwd < bwd


def test_helpers_follow_the_source_hash():
    # both readers return values only for a summary taken on the current source
    current = bench.kernel_source_hash()
    traffic_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", _text(bench.TRAFFIC_FILE)).group(1)
    trace_hash = re.search(r"sha256 \(first 16 hex\): `([0-9a-f]+)`", _text(bench.TRACE_FILE)).group(1)
    assert (bench.measured_traffic() is not None) == (traffic_hash == current)
    assert (bench.traced_durations() is not None) == (trace_hash == current)


def test_single_gpu_only(tmp_path):
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and '"error"' in res.stdout
