"""CPU-side checks of bench.py's command line: it measures one GPU and says so, without touching a device,
when asked for more; every workload it names is one its argument parser accepts."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n), "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stderr
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""  # no JSON line: nothing was measured


def test_help_lists_the_default_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert "decode_1m_hierarchical" in r.stdout
