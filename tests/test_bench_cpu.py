"""CPU checks of the benchmark's contract: one GPU only, and its algorithmic FLOP accounting.

The per-configuration totals below were derived independently (by hand, from the work each step
of the layer must do: the projection 2Nd(e+s) plus the gate 2Nde, the causal local term
N(c+1)(s+e) or 2Nc(s+e), the chunk summaries and read-outs 2·2N′se with N′ = N − Bc when causal,
the output projection 2Ned) and are restated here as numbers, so that a slip in bench.alg_flops
(a dropped term, the causal half, the first chunk's empty read-out) changes a total.
"""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("args,gflop", [
    ((1, 512, 256, 512, 128, 128, False), 0.65),
    ((4, 1024, 512, 1024, 128, 256, True), 16.25),
    ((8, 4096, 768, 1536, 128, 256, True), 276.54),
    ((2, 8192, 768, 1536, 128, 256, True), 138.67),
    ((2, 8192, 768, 1536, 128, 512, True), 145.25),
    ((2, 8192, 768, 1536, 128, 256, False), 146.03),
    ((2, 8192, 768, 1536, 128, 512, False), 159.99),
    ((1, 32768, 1024, 2048, 128, 512, True), 491.31),
])
def test_algorithmic_flops_per_workload(args, gflop):
    flops = _bench().alg_flops(*args)
    assert round(sum(flops.values()) / 1e9, 2) == gflop
    assert flops["pack"] == 0 and flops["carry"] == 0  # data movement only


def test_headline_flops_split():
    # n = 4096, B = 8: projection of V and Z, the gate's GEMM inside mix, the output projection
    B, n, d, e, s, c = 8, 4096, 768, 1536, 128, 256
    N = B * n
    f = _bench().alg_flops(B, n, d, e, s, c, True)
    assert f["proj"] == 2 * N * d * (e + s)
    assert f["out"] == 2 * N * e * d
    assert f["mix"] == 2 * N * d * e + N * (c + 1) * e + 2 * (N - B * c) * s * e
    assert f["scores_states"] == N * (c + 1) * s + 2 * (N - B * c) * s * e


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_measured_traffic_needs_matching_workload_and_sources():
    b = _bench()
    assert b.measured_traffic("mix", "c2_causal_bf16_n1024") is None
    text = open(b.PROFILE_BYTES).read()
    if f"library source sha256: {b.forward_source_sha()}" in text:
        assert b.measured_traffic("mix", "c3_causal_bf16_n4096") > 0
    else:
        assert b.measured_traffic("mix", "c3_causal_bf16_n4096") is None
