"""Host-side checks of the benchmark script (no GPU): its one-GPU guard, the
fused projections it launches, and the committed traffic record it reports."""
import importlib.util
import os
import subprocess
import sys

import pytest

from sparse_linear_layers_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_projections_cover_each_linear_once(bench):
    dims = {name: (N, K) for name, N, K in synth.QWEN05B_LINEARS}
    members = [mn for _, ms, _, in bench.PROJECTIONS for mn in ms]
    assert sorted(members) == sorted(dims)
    for pname, ms, xn in bench.PROJECTIONS:
        assert len({dims[mn][1] for mn in ms}) == 1, pname  # one input width per projection


def test_traffic_record_matches_the_projections_and_sources(bench):
    """The committed counter record has one entry per launched projection,
    its algorithmic bytes follow the roofline's formula, and its source hash
    is that of the current product kernel (else the bench reports null)."""
    T = synth.QWEN05B_PREFILL_TOKENS
    dims = {name: (N, K) for name, N, K in synth.QWEN05B_LINEARS}
    rec = bench.load_traffic("prefill_products", bench.kernel_sha("gemm.hip", "sbl_device.h"))
    assert rec is not None, "profiles/traffic.json is stale: re-take the FETCH/WRITE counters"
    shapes = rec["per_shape"]
    assert list(shapes) == [p for p, _, _ in bench.PROJECTIONS]
    for pname, ms, _ in bench.PROJECTIONS:
        N = sum(dims[mn][0] for mn in ms)
        K = dims[ms[0]][1]
        alg = T * K + N * K / 4 + 4 * N + 4 * T + 4 * T * N
        assert shapes[pname]["algorithmic_bytes"] == round(alg), pname
        meas = shapes[pname]["fetch_bytes"] + shapes[pname]["write_bytes"]
        assert 0.9 * alg <= meas <= 1.2 * alg, pname  # no large re-reads or rewrites
    mean_alg = sum(v["algorithmic_bytes"] for v in shapes.values()) / len(shapes)
    assert abs(rec["algorithmic_bytes_per_launch"] - mean_alg) <= 1
