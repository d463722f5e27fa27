"""Host-side parts of bench.py (no GPU): the one-GPU guard, the traffic
lookup's source-hash check, and the oracle baseline record."""
import json
import os
import pathlib
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from flashattention_forward_fa_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_needs_the_current_kernel_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for rel in bench.KERNEL_SOURCES:   # the hash reads the sources under ROOT
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(pathlib.Path(ROOT, rel).read_bytes())
    h = bench.kernel_source_hash()
    (prof / "fa_fwd_w.pmc.txt").write_text(
        f"header\nkernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 12345\n")
    assert bench.traffic_from_profile("w") == 12345.0
    (prof / "fa_fwd_w.pmc.txt").write_text(
        "kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 12345\n")
    assert bench.traffic_from_profile("w") is None
    assert bench.traffic_from_profile("missing") is None


@pytest.mark.parametrize("backward", [False, True])
def test_cpu_baseline_record(backward):
    w = wl.make_fixed(1, 2, 64, 64, 64, seed=5, causal=True, name="tiny")
    rec = bench.cpu_baseline(w, 0.0, backward)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and isinstance(rec["cpu"], str)
    assert rec["sample"].startswith("1 of 2 ")
    json.dumps(rec)
