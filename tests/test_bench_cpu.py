"""Host-side behaviour of bench.py that needs no GPU: the one-GPU rule, the
kernel-source gate on stored HBM traffic, and the agreement between the
committed profile summaries and the figures bench.py reads from them."""
from __future__ import annotations

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def _traffic_file(tmp_path, h, value):
    p = tmp_path / "traffic.txt"
    p.write_text(f"traffic_bytes_per_launch: {value}\nkernel_source_sha256: {h}\n")
    return str(p)


def test_stored_traffic_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    good = _traffic_file(tmp_path, bench.kernel_source_hash(), 541639051)
    monkeypatch.setattr(bench, "traffic_profile_path", lambda w: good)
    assert bench.stored_traffic("gqa_32x4096") == 541639051.0
    stale = _traffic_file(tmp_path, "0123456789abcdef", 541639051)
    monkeypatch.setattr(bench, "traffic_profile_path", lambda w: stale)
    assert bench.stored_traffic("gqa_32x4096") is None
    monkeypatch.setattr(bench, "traffic_profile_path", lambda w: str(tmp_path / "missing.txt"))
    assert bench.stored_traffic("gqa_32x4096") is None


def test_kernel_source_hash_covers_the_build_flags():
    names = [os.path.basename(p) for p in bench.KERNEL_SOURCES]
    assert "decode_kernels.hip" in names and "build.py" in names
    for p in bench.KERNEL_SOURCES:
        assert os.path.exists(p), p


@pytest.mark.parametrize("workload", bench.BENCH_WORKLOADS)
def test_profile_summaries_are_self_consistent(workload):
    """Each traffic summary's total is its read plus write bytes, and its
    ratio is that total over the algorithmic bytes it states; the kernel
    trace summary of the same workload carries the same source hash."""
    kind = "multi_token" if workload in bench.MULTI_TOKEN_WORKLOADS else "decode"
    tpath = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.txt")
    kpath = os.path.join(ROOT, "profiles", f"{kind}_{workload}_kernel_trace.txt")
    assert os.path.exists(tpath) and os.path.exists(kpath)
    t = open(tpath).read()
    rd = float(re.search(r"-> (\d+) B read per launch", t).group(1))
    wr = float(re.search(r"-> (\d+) B written per launch", t).group(1))
    total = float(re.search(r"traffic_bytes_per_launch: (\d+)", t).group(1))
    alg = float(re.search(r"algorithmic KV bytes per launch in the profiled step: (\d+)", t).group(1))
    ratio = float(re.search(r"traffic / algorithmic = ([0-9.]+)", t).group(1))
    assert abs(rd + wr - total) <= 2
    assert abs(total / alg - ratio) < 1e-3
    h_t = re.search(r"kernel_source_sha256: (\w+)", t).group(1)
    h_k = re.search(r"kernel_source_sha256: (\w+)", open(kpath).read()).group(1)
    assert h_t == h_k
