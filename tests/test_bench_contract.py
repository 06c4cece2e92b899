"""bench.py's contract pieces that run without a GPU: it measures one GPU
and refuses other counts before touching the device, and it reports the
committed counter traffic of the roofline kernel only while that record was
taken on the current kernel sources."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_quant_gemm_amd import build  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_reported_only_for_current_sources(monkeypatch):
    t = bench.measured_traffic(bench.KFN["gmm"])
    if t is None:
        pytest.skip("the committed counter record predates the current kernel sources")
    assert t > 0
    monkeypatch.setattr(build, "source_digest", lambda: "0" * 64)
    assert bench.measured_traffic(bench.KFN["gmm"]) is None
    monkeypatch.undo()
    assert bench.measured_traffic("no_such_kernel") is None
