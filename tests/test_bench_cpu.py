"""CPU checks of the benchmark's contract: one GPU only, and its algorithmic FLOP and byte
accounting.

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


# Algorithmic bytes, one shape per code path of the cross-chunk sum. The totals are element counts
# worked out by hand from what each kernel must read and write on that path (restated here as
# numbers): scores read Q_quad and K_quad (2Ns) and write P's causal triangle c(c+1)/2 or c² per
# chunk; the states stage reads K_lin and V of every chunk whose summary is used (causal: all but
# each sequence's last) and writes, depending on the path, every chunk's in-group prefix, the
# chunk or group totals, or the sequence total; the carry stage reads those totals and writes or
# updates the states; mix reads V, P, Q_lin and the states of the chunks with a global term, X and
# W_u, and writes Y.
SMALL = (2, 1024, 64, 128, 32, 64)  # B, n, d, e, s, chunk: N = 2048, 16 chunks of 64, e*s = 4096


@pytest.mark.parametrize("causal,ng,branch,ss,carry,mix", [
    # causal, 4 groups of 4 chunks: prefixes B*G*es + group totals B*(ng-1)*es; carry reads those
    # totals and updates chunks 4..15 in place
    (True, 4, "groups", 131072 + 66560 + 307200 + 131072 + 24576, 24576 + 2 * 2 * 12 * 4096,
     262144 + 66560 + 61440 + 122880 + 131072 + 8192 + 262144),
    # causal, one chunk per group: chunk totals of chunks 0..14, carry writes all 16 states
    (True, 16, "chunk_per_group", 131072 + 66560 + 307200 + 2 * 15 * 4096, 2 * 15 * 4096 + 2 * 16 * 4096,
     262144 + 66560 + 61440 + 122880 + 131072 + 8192 + 262144),
    # causal, one group: the states stage writes every state, no carry launch
    (True, 1, "one_group", 131072 + 66560 + 307200 + 2 * 16 * 4096, 0,
     262144 + 66560 + 61440 + 122880 + 131072 + 8192 + 262144),
    # non-causal, one group: the sequence total only
    (False, 1, "one_group", 131072 + 131072 + 327680 + 2 * 4096, 0,
     262144 + 131072 + 65536 + 8192 + 131072 + 8192 + 262144),
    # non-causal, 4 groups: group totals, summed by the carry stage
    (False, 4, "noncausal_groups", 131072 + 131072 + 327680 + 2 * 4 * 4096, 2 * 4 * 4096 + 2 * 4096,
     262144 + 131072 + 65536 + 8192 + 131072 + 8192 + 262144),
])
def test_algorithmic_bytes_per_state_branch(causal, ng, branch, ss, carry, mix):
    b = _bench()
    B, n, d, e, s, c = SMALL
    assert b.state_branch(B, n, c, causal, ng) == branch
    got = b.alg_bytes(B, n, d, e, s, c, causal, 2, ng)
    assert got["scores_states"] == 2 * ss
    assert got["carry"] == 2 * carry
    assert got["mix"] == 2 * mix


def test_algorithmic_bytes_single_causal_chunk():
    # chunk = n, causal: no global term; the scores write the n(n+1)/2 triangle, nothing else moves
    b = _bench()
    B, n, d, e, s = 2, 1024, 64, 128, 32
    assert b.state_branch(B, n, n, True, 1) == "none"
    got = b.alg_bytes(B, n, d, e, s, n, True, 2, 1)
    assert got["scores_states"] == 2 * (2 * 2048 * 32 + 2 * (1024 * 1025 // 2))
    assert got["carry"] == 0
    assert got["mix"] == 2 * (262144 + 2 * 524800 + 131072 + 8192 + 262144)


def test_headline_bytes():
    # n = 4096, B = 8, causal bf16, 16 chunks per sequence in 16 groups of one
    b = _bench()
    got = b.alg_bytes(8, 4096, 768, 1536, 128, 256, True, 2, 16)
    assert got == {"pack": 14548992, "proj": 187105280, "scores_states": 174620672,
                   "carry": 97517568, "mix": 317489152, "out": 153354240}


def test_committed_counters_cover_the_algorithmic_bytes():
    # The copy-calibrated HBM traffic of every kernel in the committed rocprofv3 summary must be at
    # least the algorithmic minimum (a model that claims more bytes than any run moved is wrong).
    b = _bench()
    alg = b.alg_bytes(8, 4096, 768, 1536, 128, 256, True, 2, 16)
    rows = {}
    for line in open(b.PROFILE_BYTES).read().splitlines():
        parts = line.split()
        if parts and parts[0] in alg and len(parts) == 6:
            rows[parts[0]] = int(parts[5])
    assert set(rows) == set(alg)
    for k, v in alg.items():
        assert rows[k] >= 0.95 * v, (k, rows[k], v)
