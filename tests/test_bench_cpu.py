"""The benchmark's host-side legs, on the CPU: the oracle baselines (layer
forward and offline pooling on forked worker processes) report the fields the
JSON line carries, and a request for more than one GPU ends with a message
and a nonzero status."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def small_decode():
    w = W.make_workload("decode-100m", bank_tokens=150_000)
    return w, W.query_inputs(w)


def test_cpu_baseline_fields(small_decode):
    w, qi = small_decode
    rec = bench.cpu_baseline(w, qi, 20, 2)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["cores"] == 2 and rec["value"] > 0
    assert "oracle.chunk_scores" in rec["sample"]


def test_cpu_pool_baseline_fields(small_decode):
    w, qi = small_decode
    rec = bench.cpu_pool_baseline(w, qi, 4, 2)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["cores"] == 2 and rec["value"] > 0
    # extrapolated linearly in the tokens to the whole bank of the workload
    assert abs(rec["extrapolated_s_whole_bank"] * rec["value"] - w.n_tok) <= 1e-6 * w.n_tok
    assert bench._CPU_JOB == {}   # the inputs the workers inherited are released


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
