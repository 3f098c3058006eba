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


def test_traffic_record_lookup(tmp_path, monkeypatch):
    """measured_traffic returns a kernel's calibrated counter bytes only for
    the recorded workload, a kernel the record holds, and unchanged sources."""
    import hashlib
    import json

    srcs = ["fft_block_toeplitz_amd/csrc/sbgemv.hip", "fft_block_toeplitz_amd/csrc/common.hpp"]
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, p), "rb").read() for p in srcs)).hexdigest()
    rec = {"workload": "Nm=5000 Nd=100 Nt=1000 mask 0x186", "sources": srcs, "sources_sha256": h,
           "kernels": {"sbgemv_n": {"traffic_bytes": 1234.4}, "sbgemv_c": {"traffic_bytes": 5678.6}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.measured_traffic(5000, 100, 1000, 0x186, "sbgemv_n") == 1234
    assert bench.measured_traffic(5000, 100, 1000, 0x186, "sbgemv_c") == 5679
    assert bench.measured_traffic(5000, 100, 1000, 0x000, "sbgemv_c") is None  # another workload
    assert bench.measured_traffic(5000, 100, 1000, 0x186, "other") is None     # not in the record
    rec["sources_sha256"] = "0" * 64                                            # sources changed since
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(5000, 100, 1000, 0x186, "sbgemv_c") is None
