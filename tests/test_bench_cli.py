"""bench.py's command line on the host: workload shapes and the one-GPU rule
(no GPU needed)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_named_and_explicit_shapes():
    main = bench.shape_of("main")
    assert (main.Nm, main.Nd, main.Nt) == (5000, 100, 1000)
    s = bench.shape_of("5000x100x1029")
    assert (s.Nm, s.Nd, s.Nt) == (5000, 100, 1029)
    for bad in ("5000x100", "0x1x1", "axbxc", "huge"):
        with pytest.raises(SystemExit):
            bench.shape_of(bad)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
