"""Host-side checks of the benchmark's contract (no GPU): the single-GPU guard, and the link between
the committed HBM-traffic profile and the kernel sources it was taken from (the bench line reports
the counters' traffic only while the sources hash to the value stored with them)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_gemv_decode_amd import profiling  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration that was not measured


def test_traffic_profile_is_used_only_for_its_sources(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: stored["kernel_source_sha256_16"])
    t = bench.load_traffic()
    assert t is not None and t["bytes_per_launch"] == stored["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic() is None


def test_traffic_profile_fields_are_consistent():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["bytes_per_launch"] == t["hbm_read_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]
    assert 0 < t["fetch_calibration"] <= 1.0 and 0 < t["write_calibration"] <= 1.0
    assert len(t["kernel_source_sha256_16"]) == 16
    int(t["kernel_source_sha256_16"], 16)
    assert "rocprofv3 --pmc FETCH_SIZE" in t["commands"] and "WRITE_SIZE" in t["commands"]


@pytest.mark.parametrize("index", range(len(profiling.KERNEL_SRCS)))
def test_source_hash_covers_every_kernel_source(tmp_path, monkeypatch, index):
    # copies of the sources; one byte appended to one of them must change the hash
    copies = []
    for i, src in enumerate(profiling.KERNEL_SRCS):
        dst = tmp_path / f"{i}_{os.path.basename(src)}"
        with open(src, "rb") as f:
            dst.write_bytes(f.read())
        copies.append(str(dst))
    monkeypatch.setattr(profiling, "KERNEL_SRCS", copies)
    before = profiling.kernel_source_hash()
    with open(copies[index], "ab") as f:
        f.write(b" ")
    assert profiling.kernel_source_hash() != before
