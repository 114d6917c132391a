"""Host-side checks of bench.py that need no GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8"])
def test_bench_refuses_several_gpus(n):
    """The layer has one-GPU kernels only: asking for more GPUs exits with
    status 2 and says why, before any device work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_traffic_figures_name_their_sources():
    """The stored HBM byte figures carry the digest of the sources they were
    measured on, and every source in that list exists."""
    sys.path.insert(0, ROOT)
    import bench
    for f in bench.TRAFFIC_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, f)), f
    assert len(bench.TRAFFIC_DIGEST) == 64
    assert set(bench.TRAFFIC_BYTES) == {"gate_up", "down_combine"}
