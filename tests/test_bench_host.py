"""Host-side checks of bench.py's contract (no GPU): the one-GPU guard, and
that the committed counter summary it reports `traffic` from is either
current for the quantize kernel's sources (then within 1% of the
algorithmic bytes, 2.5625 B per element) or ignored."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_traffic_figure_matches_sources_or_is_dropped():
    numel = 32768 * 5120
    t = bench.measured_traffic(numel)
    if t is not None:
        assert abs(t - numel * bench.BYTES_PER_ELEM) <= 0.01 * numel * bench.BYTES_PER_ELEM
    assert bench.measured_traffic(numel + 16) is None  # another size: no figure


def test_kernel_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16
