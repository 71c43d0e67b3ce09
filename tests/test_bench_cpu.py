"""bench.py's host logic, on the CPU: the algorithmic byte and flop counts behind the rooflines,
the rule that measured traffic is used only for the kernel source it was taken on, and the
one-GPU guard."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

from selective_state_space_conv1d_amd.synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_counts_at_the_ultra_layer(bench):
    dp, dd = WORKLOADS["prefill_ultra_8k"], WORKLOADS["decode_ultra_b64"]
    L, H, P, G, N = 8192, 256, 64, 8, 128
    # scan: x and y (bf16), B and C (bf16), dt (bf16) per token, the fp32 final state once
    assert bench.scan_bytes(dp) == L * (2 * H * P * 2 + 2 * G * N * 2 + H * 2) + H * P * N * 4 == 583008256
    # flops: C.B^T per group and chunk, scores x X, C.H and the chunk state per head
    Q = 128
    assert bench.scan_flops(dp) == L * (2 * H * P * (Q + 2 * N) + 2 * G * Q * N)
    # decode update: the fp32 state read and written, one token of x, B, C, dt in and y out
    state = 64 * H * P * N * 4
    assert bench.update_bytes(dd) == 2 * state + 64 * (2 * H * P + 2 * G * N + H) * 2 == 1078231040
    # conv: every channel in and out once (bf16), taps and bias, the conv state out
    CD = H * P + 2 * G * N
    assert bench.conv_bytes(dp, L) == L * CD * 4 + CD * 10 + CD * 8
    # the packed scan adds the initial states it reads and the final states it writes
    assert bench.varlen_scan_bytes(dp, L, 12, 24) - (bench.scan_bytes(dp) - H * P * N * 4) == 36 * H * P * N * 4


def test_traffic_is_used_only_for_the_source_it_was_measured_on(bench, tmp_path, monkeypatch):
    sha = bench.source_sha("chunk_scan")
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernels": {"chunk_scan": {"source_sha": sha, "bytes_per_launch": 6.0e8}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("chunk_scan") == 6.0e8
    assert bench.traffic_rate("chunk_scan", 1e-3) == pytest.approx(600.0)
    f.write_text(json.dumps({"kernels": {"chunk_scan": {"source_sha": "0" * 16, "bytes_per_launch": 6.0e8}}}))
    assert bench.measured_traffic("chunk_scan") is None and bench.traffic_rate("chunk_scan", 1e-3) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("chunk_scan") is None


def test_committed_traffic_matches_the_current_sources(bench):
    """profiles/hbm_traffic.json was taken on the kernel sources in the tree, so the bench's
    roofline carries measured traffic."""
    for k in ("chunk_scan", "state_update", "conv1d_fwd"):
        assert bench.measured_traffic(k) is not None, k


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
