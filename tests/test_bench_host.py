"""bench.py's host-side logic, without a GPU: it refuses more than one GPU
before touching torch, and the committed HBM-traffic record it reports is
keyed to the forward kernel's sources and agrees with the algorithmic bytes
of prefill_8k."""

import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and "multi-GPU" in r.stderr


def test_traffic_record_is_keyed_to_the_kernel_sources():
    b = _bench()
    with open(b.TRAFFIC_FILE) as f:
        rec = json.load(f)
    for key in ("kernel_sha256", "bytes_per_launch", "fetch_bytes", "write_bytes", "fetch_factor", "write_factor"):
        assert key in rec, key
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    got = b._traffic(None)
    if got is None:
        pytest.skip("the forward kernel's sources changed since the counters were taken: the bench reports null")
    assert got == rec["bytes_per_launch"]
    # prefill_8k: Q, K, V read once (3 x 32 x 8192 x 128 bf16), O bf16 and L fp32 written once
    reads = 3 * 32 * 8192 * 128 * 2
    writes = 32 * 8192 * 128 * 2 + 32 * 8192 * 4
    assert 1.0 <= rec["fetch_bytes"] / reads < 1.05
    assert 1.0 <= rec["write_bytes"] / writes < 1.05
