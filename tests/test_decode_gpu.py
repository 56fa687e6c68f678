"""GPU parity of the causal decoding step (flash_gau_decode_step through the C ABI) against the
oracle's decode_step on identical inputs, step by step.

Error measure per step: max |o_gpu - o_ref| / max |o_ref|; bar 2e-2 for bf16, 1e-4 for fp32. The
carried fp32 state and the chunk cache are compared too. Every state buffer starts filled with
0xFF bytes (NaN in both element types): the step at t = 0 must clear what it reads.
"""

import numpy as np
import pytest

import oracle
from efficient_transformer_attention_amd import flashgau as fg
from efficient_transformer_attention_amd import inputs as gen

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}

# name: (B, d, e, s, chunk, steps T, normalising n, dtype, gamma_std, beta_std)
CASES = {
    "small_bf16": (3, 64, 136, 24, 8, 19, 32, "bf16", 0.3, 0.1),
    "small_f32": (3, 64, 136, 24, 8, 19, 32, "f32", 0.3, 0.1),
    "batch17_ktail_bf16": (17, 40, 88, 16, 4, 9, 16, "bf16", 0.3, 0.1),
    "chunk1_f32": (2, 32, 64, 8, 1, 5, 5, "f32", 0.3, 0.1),
    "wide_chunk_f32": (2, 48, 264, 40, 40, 43, 80, "f32", 0.3, 0.1),
    # two K tiles of the matrix-core fold, the second ragged (72 = 64 + 8 tokens); two folds
    "ragged_fold_bf16": (2, 48, 264, 40, 72, 150, 160, "bf16", 0.3, 0.1),
    "n4096_dims_bf16": (8, 768, 1536, 128, 256, 300, 4096, "bf16", 0.02, 0.0),
}


def _torch():
    import torch
    return torch


def _dev(a, dtype):
    torch = _torch()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(tdt).contiguous()


def _rel(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def _inputs(B, d, e, s, chunk, T, dtype, gstd, bstd, seed=0):
    n_gen = -(-T // chunk) * chunk
    return gen.make_inputs(B, n_gen, d, e, s, chunk, True, dtype, seed=seed, gamma_std=gstd, beta_std=bstd)


def run_decode_gpu(inp, T, n, dtype):
    torch = _torch()
    B, _, d, e, s = inp.shape
    W = [_dev(w, dtype) for w in (inp.W_u, inp.W_v, inp.W_z, inp.W_o)]
    gamma, beta = _dev(inp.gamma, "f32"), _dev(inp.beta, "f32")
    packed = fg.pack_weights(*W)
    state = fg.DecodeState(B, d, e, s, inp.chunk, W[0].dtype, "cuda")
    state.buf.fill_(255)
    X = _dev(inp.X, dtype)
    outs = []
    for t in range(T):
        o = fg.flash_gau_decode_step(X[:, t].contiguous(), packed, gamma, beta, inp.chunk, t, n, state)
        outs.append(o.float())
    torch.cuda.synchronize()
    O = torch.stack(outs, 1).cpu().numpy().astype(np.float64)
    views = {k: v.float().cpu().numpy().astype(np.float64) for k, v in state.views().items()}
    return O, views


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_steps_match_oracle(name):
    B, d, e, s, chunk, T, n, dtype, gstd, bstd = CASES[name]
    print(f"[gpu case] decode {name} B={B} d={d} e={e} s={s} c={chunk} T={T}", flush=True)
    inp = _inputs(B, d, e, s, chunk, T, dtype, gstd, bstd)
    got, views = run_decode_gpu(inp, T, n, dtype)
    ref, state = oracle.decode_sequence(inp.X[:, :T], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta,
                                        inp.W_o, chunk, n=n)
    assert np.isfinite(got).all()
    errs = [_rel(got[:, t], ref[:, t]) for t in range(T)]
    worst = int(np.argmax(errs))
    print(f"[gpu case] decode {name}: worst step {worst} rel err {errs[worst]:.3e}", flush=True)
    assert errs[worst] <= TOL[dtype], (worst, errs[worst])
    # the carried state (fp32 on both sides) and the cache rows of the current chunk
    assert _rel(views["S"], state["S"]) <= TOL[dtype]
    i = (T - 1) % chunk
    for k, ko in (("KQ", "Kq"), ("KL", "Kl"), ("V", "V")):
        assert _rel(views[k][:, : i + 1], state[ko][:, : i + 1]) <= TOL[dtype], k


def test_decode_agrees_with_gpu_forward_rows():
    # both GPU paths on one input: stepping t = 0..n-1 reproduces the causal forward's rows
    torch = _torch()
    B, n, d, e, s, chunk, dtype = 2, 48, 64, 96, 24, 16, "bf16"
    print("[gpu case] decode vs forward rows", flush=True)
    inp = gen.make_inputs(B, n, d, e, s, chunk, True, dtype, seed=4, gamma_std=0.3, beta_std=0.1)
    got, _ = run_decode_gpu(inp, n, n, dtype)
    args = [_dev(inp.X, dtype), _dev(inp.W_u, dtype), _dev(inp.W_v, dtype), _dev(inp.W_z, dtype),
            _dev(inp.gamma, "f32"), _dev(inp.beta, "f32"), _dev(inp.W_o, dtype)]
    O = fg.flash_gau_forward(*args, chunk, True)
    torch.cuda.synchronize()
    fwd = O.float().cpu().numpy().astype(np.float64)
    ref = oracle.flash_forward(inp.X, inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o, chunk, True)
    assert _rel(fwd, ref) <= TOL[dtype]
    assert _rel(got, ref) <= TOL[dtype]
    assert _rel(got, fwd) <= 2 * TOL[dtype]


def test_packed_weights_are_the_transposes():
    torch = _torch()
    d, e, s = 40, 88, 16
    print("[gpu case] pack weights", flush=True)
    inp = gen.make_inputs(1, 8, d, e, s, 8, True, "bf16", seed=2)
    W = [_dev(w, "bf16") for w in (inp.W_u, inp.W_v, inp.W_z, inp.W_o)]
    packed = fg.pack_weights(*W)
    torch.cuda.synchronize()
    wcat = packed[: (2 * e + s) * d * 2].view(torch.bfloat16).view(2 * e + s, d).float().cpu().numpy()
    wo_off = ((2 * e + s) * d * 2 + 255) // 256 * 256
    wo = packed[wo_off: wo_off + d * e * 2].view(torch.bfloat16).view(d, e).float().cpu().numpy()
    want = np.concatenate([inp.W_u, inp.W_v, inp.W_z], axis=1).T
    assert np.array_equal(wcat, want.astype(np.float32))
    assert np.array_equal(wo, inp.W_o.T.astype(np.float32))


def test_decode_is_deterministic():
    B, d, e, s, chunk, T, n, dtype, gstd, bstd = CASES["small_bf16"]
    print("[gpu case] decode determinism", flush=True)
    inp = _inputs(B, d, e, s, chunk, T, dtype, gstd, bstd, seed=7)
    a, _ = run_decode_gpu(inp, T, n, dtype)
    b, _ = run_decode_gpu(inp, T, n, dtype)
    assert np.array_equal(a, b)


def test_decode_steps_replayed_from_a_hip_graph_match_eager():
    # Steps t0..t1-1 captured once into a HIP graph (torch.cuda.CUDAGraph); before each replay the
    # state is restored eagerly from a saved copy; every replay must give the eager outputs bitwise.
    torch = _torch()
    B, d, e, s, c, n, dtype = 3, 64, 136, 24, 8, 32, "bf16"
    t0, t1 = 6, 19  # crosses a chunk end (the fold after t = 15)
    print("[gpu case] decode graph replay", flush=True)
    inp = _inputs(B, d, e, s, c, 24, dtype, 0.3, 0.1, seed=9)
    W = [_dev(w, dtype) for w in (inp.W_u, inp.W_v, inp.W_z, inp.W_o)]
    gamma, beta = _dev(inp.gamma, "f32"), _dev(inp.beta, "f32")
    packed = fg.pack_weights(*W)
    X = _dev(inp.X, dtype)
    xs = [X[:, t].contiguous() for t in range(t1)]
    state = fg.DecodeState(B, d, e, s, c, W[0].dtype, "cuda")
    for t in range(t0):
        fg.flash_gau_decode_step(xs[t], packed, gamma, beta, c, t, n, state)
    torch.cuda.synchronize()
    saved = state.buf.clone()
    outs = [torch.empty((B, d), dtype=W[0].dtype, device="cuda") for _ in range(t0, t1)]
    eager = [fg.flash_gau_decode_step(xs[t], packed, gamma, beta, c, t, n, state).clone()
             for t in range(t0, t1)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    state.buf.copy_(saved)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for k, t in enumerate(range(t0, t1)):
            fg.flash_gau_decode_step(xs[t], packed, gamma, beta, c, t, n, state, out=outs[k],
                                     stream=stream.cuda_stream)
    for rep in range(3):
        state.buf.copy_(saved)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in range(len(outs)):
            assert torch.equal(outs[k], eager[k]), (rep, k)
