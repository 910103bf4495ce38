"""CPU checks of bench.py's contract: the one-GPU guard and the rule that
measured HBM traffic is reported only for the kernel source it was measured
on."""

import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in res.stderr and f"--gpus {n}" in res.stderr
    assert res.stdout.strip() == ""  # no JSON line


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    bench = load_bench()
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"prefill_x": {"bytes_per_launch": 1234, "kernel_source_sha256_16": "aaaa"}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "aaaa")
    assert bench.measured_traffic("prefill_x") == 1234
    assert bench.measured_traffic("decode_y") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "bbbb")
    assert bench.measured_traffic("prefill_x") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "aaaa")
    assert bench.measured_traffic("prefill_x") is None


def test_kernel_source_hash_is_the_kernel_file_digest():
    import hashlib
    bench = load_bench()
    with open(os.path.join(ROOT, "long_context_serving_amd", "csrc", "kernels.hip"), "rb") as fh:
        want = hashlib.sha256(fh.read()).hexdigest()[:16]
    assert bench.kernel_source_hash() == want
