"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on identical inputs.

Error measure: max |O_gpu - O_ref| / max |O_ref| per tensor; bar 2e-2 for bf16 and 1e-4 for fp32.
The global linear branch dominates the output's magnitude at the workload distributions, so each
branch is also checked on its own (the other head switched off), and every intermediate the
library leaves in its workspace is compared with the oracle's.
"""

import numpy as np
import pytest

import oracle
from efficient_transformer_attention_amd import flashgau as fg
from efficient_transformer_attention_amd import inputs as gen

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _torch():
    import torch
    return torch


def _dev(a, dtype):
    torch = _torch()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(tdt).contiguous()


def _rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def run_gpu(inp, views=False):
    """Runs the library on `inp`; returns O as float64 numpy and optionally workspace views."""
    torch = _torch()
    B, n, d, e, s = inp.shape
    dt = fg.BF16 if inp.dtype == "bf16" else fg.F32
    args = [_dev(inp.X, inp.dtype), _dev(inp.W_u, inp.dtype), _dev(inp.W_v, inp.dtype),
            _dev(inp.W_z, inp.dtype), _dev(inp.gamma, "f32"), _dev(inp.beta, "f32"),
            _dev(inp.W_o, inp.dtype)]
    nbytes = fg.workspace_size(B, n, d, e, s, inp.chunk, inp.causal, dt)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device="cuda")
    O = fg.flash_gau_forward(*args, inp.chunk, inp.causal, workspace=ws)
    torch.cuda.synchronize()
    out = O.float().cpu().numpy().astype(np.float64)
    if not views:
        return out
    v = fg.workspace_views(ws, B, n, d, e, s, inp.chunk, inp.causal, dt)
    # CARRY holds only what the carry stage reads (nothing with one chunk group per sequence)
    return out, {k: t.float().cpu().numpy().astype(np.float64) for k, t in v.items() if k != "CARRY"}


def run_oracle(inp, batches=None, intermediates=False):
    X = inp.X if batches is None else inp.X[batches]
    return oracle.flash_forward(X, inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o,
                                inp.chunk, inp.causal, return_intermediates=intermediates)


def _announce(name):
    print(f"[gpu case] {name}", flush=True)


SMALL = {
    # name: (B, n, d, e, s, chunk, causal, dtype)
    "c1_noncausal_fp32": gen.WORKLOADS["c1_noncausal_fp32_n512"],
    "c2_causal_bf16": gen.WORKLOADS["c2_causal_bf16_n1024"],
    "c2_noncausal_bf16": (4, 1024, 512, 1024, 128, 256, False, "bf16"),
    "c1_causal_fp32": (1, 512, 256, 512, 128, 128, True, "f32"),
    "ragged_causal_bf16": (2, 216, 200, 136, 24, 72, True, "bf16"),
    "ragged_noncausal_bf16": (2, 216, 200, 136, 24, 72, False, "bf16"),
    "ragged_causal_fp32": (2, 216, 200, 136, 24, 72, True, "f32"),
    "ragged_noncausal_fp32": (3, 144, 40, 88, 136, 48, False, "f32"),
    "chunk_eq_n_causal_bf16": (2, 256, 128, 256, 128, 256, True, "bf16"),
    "chunk_eq_n_noncausal_fp32": (2, 192, 64, 128, 128, 192, False, "f32"),
    "tiny_causal_bf16": (1, 8, 8, 8, 8, 8, True, "bf16"),
    "tiny_noncausal_fp32": (1, 16, 8, 16, 8, 8, False, "f32"),
    "many_chunks_causal_bf16": (2, 1024, 64, 128, 128, 8, True, "bf16"),
    "wide_chunk_c512_causal_bf16": (1, 1536, 256, 512, 128, 512, True, "bf16"),
    # the states stage's chunk grouping (flashgau_state_groups): two chunks per group, so the
    # carry walk adds earlier groups' totals to in-group prefixes; and one group per sequence
    # (B * state tiles >= 2048), where the states stage writes every state and no carry runs
    "chunk_groups_causal_bf16": (8, 256, 64, 1536, 16, 8, True, "bf16"),
    "chunk_groups_noncausal_bf16": (8, 256, 64, 1536, 16, 8, False, "bf16"),
    "one_group_causal_bf16": (128, 64, 32, 2048, 128, 16, True, "bf16"),
    "one_group_noncausal_bf16": (128, 64, 32, 2048, 128, 16, False, "bf16"),
    "one_group_causal_fp32": (128, 64, 32, 2048, 128, 16, True, "f32"),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_parity_end_to_end(name):
    B, n, d, e, s, c, causal, dtype = SMALL[name]
    _announce(name)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=1, beta_std=0.1)
    got = run_gpu(inp)
    ref = run_oracle(inp)
    err = _rel(got, ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("branch", ["local", "linear"])
@pytest.mark.parametrize("name", ["c2_causal_bf16", "c2_noncausal_bf16", "ragged_causal_fp32",
                                  "wide_chunk_c512_causal_bf16"])
def test_parity_each_branch(name, branch):
    B, n, d, e, s, c, causal, dtype = SMALL[name]
    _announce(f"{name} {branch} only")
    inp = gen.isolate_branch(gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=2, beta_std=0.1),
                             branch)
    err = _rel(run_gpu(inp), run_oracle(inp))
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("name", ["c2_causal_bf16", "c2_noncausal_bf16", "ragged_causal_bf16",
                                  "ragged_noncausal_fp32", "c1_noncausal_fp32",
                                  "chunk_groups_causal_bf16", "chunk_groups_noncausal_bf16",
                                  "one_group_causal_bf16", "one_group_noncausal_bf16"])
def test_stage_parity(name):
    B, n, d, e, s, c, causal, dtype = SMALL[name]
    _announce(f"{name} stages")
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=3, beta_std=0.1)
    O, v = run_gpu(inp, views=True)
    O_ref, it = run_oracle(inp, intermediates=True)
    G = n // c
    tol = TOL[dtype]
    lower = np.tril(np.ones((c, c), dtype=bool))
    checks = {
        "V": (v["VT"].reshape(B, G, e, c).transpose(0, 1, 3, 2).reshape(B, n, e), it["V"]),
        "Q_quad": (v["QQ"].reshape(B, n, s), it["Qq"]),
        "K_quad": (v["KQ"].reshape(B, n, s), it["Kq"]),
        "Q_lin": (v["QL"].reshape(B, n, s), it["Ql"]),
        "K_lin": (v["KLT"].reshape(B, G, s, c).transpose(0, 1, 3, 2).reshape(B, n, s), it["Kl"]),
        # causal: blocks above the diagonal are left unwritten; the lower triangle is compared
        "P": ((np.where(lower, v["P"].reshape(B, G, c, c), 0.0), it["P"]) if causal
              else (v["P"].reshape(B, G, c, c), it["P"])),
        "Y": (v["Y"].reshape(B, n, e), it["Y"]),
        "O": (O, O_ref),
    }
    S_ref = it["S"] / n  # [B, G, s, e]
    if causal:
        checks["S"] = (v["ST"].reshape(B, G, e, s).transpose(0, 1, 3, 2), S_ref)
    else:
        checks["S"] = (v["ST"].reshape(B, 1, e, s).transpose(0, 1, 3, 2), S_ref[:, :1])
    for key, (got, ref) in checks.items():
        err = _rel(got, ref)
        print(f"  {key:7s} max rel err {err:.3e}", flush=True)
        assert err <= tol, key
    if causal:
        # the first chunk of every sequence reads an empty prefix
        assert np.all(v["ST"].reshape(B, G, e, s)[:, 0] == 0.0)


@pytest.mark.parametrize("name,t", [("c2_causal_bf16", 300), ("ragged_causal_fp32", 100),
                                    ("many_chunks_causal_bf16", 517),
                                    ("c3_causal_bf16_n4096", 2900)])
def test_causal_output_ignores_future_tokens(name, t):
    # (the last case runs the headline configuration at full size)
    B, n, d, e, s, c, causal, dtype = SMALL[name] if name in SMALL else gen.WORKLOADS[name]
    _announce(f"{name} causality t={t}")
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=4)
    O1 = run_gpu(inp)
    X2 = inp.X.copy()
    X2[:, t:] = gen.round_to(np.random.default_rng(5).standard_normal(X2[:, t:].shape) * 2, dtype)
    import dataclasses
    O2 = run_gpu(dataclasses.replace(inp, X=X2))
    assert np.array_equal(O1[:, :t], O2[:, :t])  # bitwise: no value from the future enters
    assert not np.array_equal(O1[:, t:], O2[:, t:])


@pytest.mark.parametrize("name", ["c2_causal_bf16", "c1_noncausal_fp32"])
def test_repeat_calls_are_bitwise_identical(name):
    B, n, d, e, s, c, causal, dtype = SMALL[name]
    _announce(f"{name} determinism")
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=6)
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert np.array_equal(a, b)


def test_empty_batch_launches_nothing():
    torch = _torch()
    _announce("empty")
    X = torch.empty((0, 256, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    Wz = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.ones((4, 128), dtype=torch.float32, device="cuda")
    Wo = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    out = fg.flash_gau_forward(X, W, W, Wz, g, g, Wo, 64, True)
    torch.cuda.synchronize()
    assert out.shape == (0, 256, 64)


def test_timed_entry_point_matches_and_orders_events():
    import ctypes
    torch = _torch()
    _announce("timed entry point")
    B, n, d, e, s, c, causal, dtype = SMALL["c2_causal_bf16"]
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=7)
    ref = run_gpu(inp)
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(len(fg.STAGES) + 1):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h.value)
    args = [_dev(a, dtype) for a in (inp.X, inp.W_u, inp.W_v, inp.W_z)]
    gamma, beta = _dev(inp.gamma, "f32"), _dev(inp.beta, "f32")
    Wo = _dev(inp.W_o, dtype)
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, fg.BF16)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, n, d), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = fg.forward_timed_raw(args[0].data_ptr(), args[1].data_ptr(), args[2].data_ptr(),
                              args[3].data_ptr(), gamma.data_ptr(), beta.data_ptr(), Wo.data_ptr(),
                              c, causal, B, n, d, e, s, fg.BF16, O.data_ptr(), ws.data_ptr(), nbytes,
                              stream, evs)
    assert rc == fg.OK
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), ref)
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    for i in range(len(evs) - 1):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[i], evs[i + 1]) == 0
        assert ms.value >= 0.0
    for h in evs:
        hip.hipEventDestroy(ctypes.c_void_p(h))
    # the per-kernel form: a start and a stop event for each kernel, the kernels in launch order
    pairs = []
    for _ in range(2 * len(fg.STAGES)):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        pairs.append(h.value)
    O.zero_()
    rc = fg.forward_timed_raw(args[0].data_ptr(), args[1].data_ptr(), args[2].data_ptr(),
                              args[3].data_ptr(), gamma.data_ptr(), beta.data_ptr(), Wo.data_ptr(),
                              c, causal, B, n, d, e, s, fg.BF16, O.data_ptr(), ws.data_ptr(), nbytes,
                              stream, pairs)
    assert rc == fg.OK
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), ref)
    for i in range(len(fg.STAGES)):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), pairs[2 * i], pairs[2 * i + 1]) == 0
        assert ms.value > 0.0  # every stage of this case launches a kernel
        if i > 0:
            assert hip.hipEventElapsedTime(ctypes.byref(ms), pairs[2 * i - 1], pairs[2 * i]) == 0
            assert ms.value >= 0.0
    bad = fg.forward_timed_raw(args[0].data_ptr(), args[1].data_ptr(), args[2].data_ptr(),
                               args[3].data_ptr(), gamma.data_ptr(), beta.data_ptr(), Wo.data_ptr(),
                               c, causal, B, n, d, e, s, fg.BF16, O.data_ptr(), ws.data_ptr(), nbytes,
                               stream, pairs[:-1])
    assert bad == fg.ERR_BAD_SHAPE
    for h in pairs:
        hip.hipEventDestroy(ctypes.c_void_p(h))


def test_timed_per_kernel_form_with_stages_that_launch_nothing():
    # chunk = n, causal: the cross-chunk stage launches nothing (the one chunk's prefix is empty);
    # its start and stop events are still recorded, back to back, and every other pair spans a kernel
    import ctypes
    torch = _torch()
    _announce("timed entry point, per kernel, single chunk")
    B, n, d, e, s, c, causal, dtype = 2, 256, 64, 128, 32, 256, True, "bf16"
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=8)
    ref = run_gpu(inp)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    pairs = []
    for _ in range(2 * len(fg.STAGES)):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        pairs.append(h.value)
    args = [_dev(a, dtype) for a in (inp.X, inp.W_u, inp.W_v, inp.W_z)]
    gamma, beta = _dev(inp.gamma, "f32"), _dev(inp.beta, "f32")
    Wo = _dev(inp.W_o, dtype)
    nbytes = fg.workspace_size(B, n, d, e, s, c, causal, fg.BF16)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, n, d), dtype=torch.bfloat16, device="cuda")
    rc = fg.forward_timed_raw(args[0].data_ptr(), args[1].data_ptr(), args[2].data_ptr(),
                              args[3].data_ptr(), gamma.data_ptr(), beta.data_ptr(), Wo.data_ptr(),
                              c, causal, B, n, d, e, s, fg.BF16, O.data_ptr(), ws.data_ptr(), nbytes,
                              torch.cuda.current_stream().cuda_stream, pairs)
    assert rc == fg.OK
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), ref)
    for i, stage in enumerate(fg.STAGES):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), pairs[2 * i], pairs[2 * i + 1]) == 0, stage
        assert ms.value >= 0.0, stage
        if stage != "carry":
            assert ms.value > 0.0, stage
    for h in pairs:
        hip.hipEventDestroy(ctypes.c_void_p(h))


def test_native_library_is_the_in_tree_build():
    import os
    _announce("library path")
    L = fg.lib()
    assert os.path.dirname(fg.LIB_PATH) == os.path.dirname(os.path.abspath(fg.__file__))
    maps = open("/proc/self/maps").read()
    assert fg.LIB_PATH in maps
    assert L is fg.lib()


# ------------------------------------------------------------------ full-size workloads (sampled)

FULL = ["c2_causal_bf16_n1024", "c3_causal_bf16_n4096", "c4_causal_bf16_n8192_c256",
        "c4_causal_bf16_n8192_c512", "c4_noncausal_bf16_n8192_c256",
        "c4_noncausal_bf16_n8192_c512", "c5_causal_bf16_n32768"]


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size_sampled_sequences(name):
    """The exact launch configuration the benchmark times, at its full size. Sequences are
    independent, so the oracle computes the first and the last sequence of the batch exactly and
    every one of their outputs is compared."""
    _announce(f"full {name}")
    inp = gen.workload_inputs(name, seed=0)
    got = run_gpu(inp)
    B = inp.X.shape[0]
    sample = sorted({0, B - 1})
    ref = run_oracle(inp, batches=sample)
    err = _rel(got[sample], ref)
    print(f"  sequences {sample}: max rel err {err:.3e}", flush=True)
    assert err <= TOL[inp.dtype]


# FLASH-Quad (chunk = n) at the long sequences the benchmark compares with FLASH: one whole
# sequence per shape, its output checked row by row against the oracle's row-wise evaluation
# (every sampled row sums relu²(q·k / n) v over all its earlier keys, up to 16384 of them).
LONG_QUAD = [(2, 8192, 1), (1, 16384, 0)]  # (B, n, sequence checked)


@pytest.mark.parametrize("B,n,seq", LONG_QUAD)
def test_flash_quad_long_sequences(B, n, seq):
    d, e, s = 768, 1536, 128
    _announce(f"flash_quad B={B} n={n} chunk=n")
    inp = gen.make_inputs(B, n, d, e, s, n, True, "bf16", seed=5, beta_std=0.1)
    O = run_gpu(inp)
    rng = np.random.default_rng(n)
    rows = sorted({0, 1, 2, n // 2, n - 2, n - 1, *rng.integers(0, n, 40).tolist()})
    ref = oracle.forward_rows(inp.X[seq], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o,
                              n, True, rows)
    assert np.isfinite(O).all()
    assert _rel(O[seq, rows], ref) <= TOL["bf16"]


def test_parity_large_output_tiles_ragged():
    # B*n = 16384 with d = 520: the output GEMM takes its 256 x 256 tiles (192 of them, one round,
    # against two rounds of 256 x 128 tiles), the last feature tile holding only 8 of 256 rows
    _announce("large output tiles, ragged d")
    inp = gen.make_inputs(1, 16384, 520, 264, 24, 256, True, "bf16", seed=9, beta_std=0.1)
    got = run_gpu(inp)
    ref = run_oracle(inp)
    assert _rel(got, ref) <= TOL["bf16"]
