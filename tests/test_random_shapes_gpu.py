"""GPU parity over seeded random shapes: the forward, the backward and the decoding step through
the C ABI against the fp64 oracle, on shapes drawn from the accepted range (every width a multiple
of 8; for the forward and backward n a multiple of the chunk), mixing element types, masks, chunk
counts and the rotary embedding, plus a few larger shapes with ragged widths. The draws are fixed by their
seeds, and each case prints its shape before it runs. Bars as in the other parity tests: max |got - ref| / max |ref| per tensor
(per step for decoding), 2e-2 for bf16, 1e-4 for fp32.
"""

import random

import numpy as np
import pytest

import oracle
from efficient_transformer_attention_amd import flashgau as fg
from efficient_transformer_attention_amd import inputs as gen

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _draw(count, seed):
    rng = random.Random(seed)
    cases = []
    for _ in range(count):
        c = 8 * rng.randint(1, 24)
        G = rng.randint(1, 4)
        B = rng.randint(1, 3)
        d, e, s = 8 * rng.randint(1, 34), 8 * rng.randint(1, 49), 8 * rng.randint(1, 25)
        dtype = rng.choice(["bf16", "f32"])
        causal = rng.random() < 0.5
        rope = rng.choice([None, 10000.0])
        cases.append((B, c * G, d, e, s, c, causal, dtype, rope))
    return cases


FORWARD = _draw(24, 11)
BACKWARD = _draw(10, 12)


def _dev(a, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(tdt).contiguous()


def _rel(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def _args(inp, dtype):
    return [_dev(inp.X, dtype), _dev(inp.W_u, dtype), _dev(inp.W_v, dtype), _dev(inp.W_z, dtype),
            _dev(inp.gamma, "f32"), _dev(inp.beta, "f32"), _dev(inp.W_o, dtype)]


@pytest.mark.parametrize("i", range(len(FORWARD)))
def test_forward_random_shape(i):
    import torch
    B, n, d, e, s, c, causal, dtype, rope = FORWARD[i]
    print(f"[gpu case] forward random shape {i}: B={B} n={n} d={d} e={e} s={s} c={c} "
          f"causal={causal} {dtype} rope={rope}", flush=True)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=100 + i, gamma_std=0.3, beta_std=0.1)
    O = fg.flash_gau_forward(*_args(inp, dtype), c, causal, rope_base=rope)
    torch.cuda.synchronize()
    ref = oracle.flash_forward(inp.X, inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o, c,
                               causal, rope_base=rope)
    err = _rel(O.float().cpu().numpy(), ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("i", range(len(BACKWARD)))
def test_backward_random_shape(i):
    import torch
    B, n, d, e, s, c, causal, dtype, rope = BACKWARD[i]
    print(f"[gpu case] backward random shape {i}: B={B} n={n} d={d} e={e} s={s} c={c} "
          f"causal={causal} {dtype} rope={rope}", flush=True)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=200 + i, gamma_std=0.3, beta_std=0.1)
    dO = gen.make_output_grad(B, n, d, dtype, seed=200 + i)
    grads = fg.flash_gau_backward(*_args(inp, dtype), _dev(dO, dtype), c, causal,
                                  rope_base=rope or 0.0)
    torch.cuda.synchronize()
    ref = oracle.flash_backward(inp.X, inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o, dO,
                                c, causal, rope_base=rope)
    errs = {k: _rel(grads[k].float().cpu().numpy(), ref[k]) for k in fg.GRAD_NAMES}
    print("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in fg.GRAD_NAMES:
        assert errs[k] <= TOL[dtype], (k, errs[k])


def _draw_decode(count, seed):
    rng = random.Random(seed)
    cases = []
    for _ in range(count):
        B = rng.randint(1, 20)
        d, e, s = 8 * rng.randint(1, 34), 8 * rng.randint(1, 49), 8 * rng.randint(1, 25)
        c = rng.randint(1, 48)
        T = rng.randint(1, min(120, 5 * c // 2 + 1))
        n = T + rng.randint(0, 64)
        cases.append((B, d, e, s, c, T, n, rng.choice(["bf16", "f32"]), rng.choice([None, 10000.0])))
    return cases


DECODE = _draw_decode(8, 13)


@pytest.mark.parametrize("i", range(len(DECODE)))
def test_decode_random_shape(i):
    # step by step from an empty state (its buffer filled with 0xFF bytes), across chunk ends
    import torch
    B, d, e, s, c, T, n, dtype, rope = DECODE[i]
    print(f"[gpu case] decode random shape {i}: B={B} d={d} e={e} s={s} c={c} T={T} n={n} {dtype} "
          f"rope={rope}", flush=True)
    inp = gen.make_inputs(B, -(-T // c) * c, d, e, s, c, True, dtype, seed=300 + i, gamma_std=0.3,
                          beta_std=0.1)
    W = [_dev(w, dtype) for w in (inp.W_u, inp.W_v, inp.W_z, inp.W_o)]
    gamma, beta = _dev(inp.gamma, "f32"), _dev(inp.beta, "f32")
    packed = fg.pack_weights(*W)
    state = fg.DecodeState(B, d, e, s, c, W[0].dtype, "cuda")
    state.buf.fill_(255)
    X = _dev(inp.X, dtype)
    outs = [fg.flash_gau_decode_step(X[:, t].contiguous(), packed, gamma, beta, c, t, n, state,
                                     rope_base=rope or 0.0).float() for t in range(T)]
    torch.cuda.synchronize()
    got = torch.stack(outs, 1).cpu().numpy().astype(np.float64)
    ref, _ = oracle.decode_sequence(inp.X[:, :T], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta,
                                    inp.W_o, c, n=n, rope_base=rope)
    errs = [_rel(got[:, t], ref[:, t]) for t in range(T)]
    worst = int(np.argmax(errs))
    print(f"  worst step {worst} rel err {errs[worst]:.3e}", flush=True)
    assert errs[worst] <= TOL[dtype], (worst, errs[worst])


# Larger shapes with ragged widths, chosen so that the large-tile paths run with partial edge
# tiles: 128 x 128 projection tiles that straddle the V | heads boundary (e not a multiple of 128),
# 256 x 256 output tiles over a d that is not a multiple of 256, chunks that are not a multiple of
# the 128-token tile, fp32's small tiles. The batch runs whole; the oracle checks its first and last
# sequence. name: (B, n, d, e, s, chunk, causal, dtype)
LARGE = {
    "straddle_c200_causal": (4, 4000, 1000, 1000, 200, 200, True, "bf16"),
    "c384_noncausal": (2, 6144, 768, 1536, 128, 384, False, "bf16"),
    "ragged8_causal": (8, 2048, 520, 1544, 136, 256, True, "bf16"),
    "long_ragged_causal": (1, 16384, 1032, 2056, 136, 512, True, "bf16"),
    "ragged_noncausal_c192": (3, 3072, 776, 1288, 200, 192, False, "bf16"),
    "fp32_ragged_causal": (2, 2048, 264, 520, 72, 128, True, "f32"),
    # wide heads: four head tiles per projection row block, a 512-deep score contraction
    "wide_heads_s512_causal": (2, 2048, 512, 1024, 512, 256, True, "bf16"),
    "wide_heads_s264_noncausal_f32": (2, 1024, 136, 264, 264, 128, False, "f32"),
}


@pytest.mark.parametrize("name", sorted(LARGE))
def test_forward_large_ragged(name):
    import torch
    B, n, d, e, s, c, causal, dtype = LARGE[name]
    print(f"[gpu case] forward large ragged {name}: B={B} n={n} d={d} e={e} s={s} c={c} "
          f"causal={causal} {dtype}", flush=True)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=400, gamma_std=0.3, beta_std=0.1)
    O = fg.flash_gau_forward(*_args(inp, dtype), c, causal)
    torch.cuda.synchronize()
    sample = sorted({0, B - 1})
    got = O.float().cpu().numpy()[sample]
    ref = oracle.flash_forward(inp.X[sample], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o,
                               c, causal)
    err = _rel(got, ref)
    print(f"  sequences {sample}: max rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("name", ["ragged8_causal", "wide_heads_s512_causal"])
def test_backward_large_ragged(name):
    # the input and weight gradients on 256 x 256 tiles with partial edge tiles in d, e and s and
    # several token ranges; dO is zero on every sequence but the first, so the oracle needs only it
    import torch
    B, n, d, e, s, c, causal, dtype = LARGE[name]
    print(f"[gpu case] backward large ragged {name}: B={B} n={n} d={d} e={e} s={s} c={c}", flush=True)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=401, gamma_std=0.3, beta_std=0.1)
    dO = gen.make_output_grad(B, n, d, dtype, seed=401)
    dO[1:] = 0.0
    grads = fg.flash_gau_backward(*_args(inp, dtype), _dev(dO, dtype), c, causal)
    torch.cuda.synchronize()
    ref = oracle.flash_backward(inp.X[:1], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o,
                                dO[:1], c, causal)
    got = {k: v.float().cpu().numpy() for k, v in grads.items()}
    assert np.abs(got["dX"][1:]).max() == 0.0
    errs = {k: _rel(got[k][:1] if k == "dX" else got[k], ref[k]) for k in fg.GRAD_NAMES}
    print("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in fg.GRAD_NAMES:
        assert errs[k] <= TOL[dtype], (k, errs[k])
