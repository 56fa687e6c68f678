"""GPU parity where buffer offsets leave 32-bit range: 2^20 tokens with e = 2056 put the
token-major intermediates (V chunk-transposed, Y, and in the backward the pre-activation gradients)
past 2^31 elements, and the fp32 case past 4 GiB. Each kernel addresses such a buffer from a 64-bit
tile base; these cases check that the last sequence, whose rows sit at the largest offsets, comes
out as the oracle computes it. The batch runs whole; the oracle runs the sampled sequences alone
(every sequence is independent). Bars as in the other parity tests: max |got - ref| / max |ref|,
2e-2 for bf16, 1e-4 for fp32.
"""

import numpy as np
import pytest

import oracle
from efficient_transformer_attention_amd import flashgau as fg
from efficient_transformer_attention_amd import inputs as gen

TOL = {"bf16": 2e-2, "f32": 1e-4}

# name: (B, n, d, e, s, chunk, causal, dtype)
CASES = {
    "bf16_2p31_elements": (1024, 1024, 64, 2056, 64, 256, True, "bf16"),
    "f32_4gib_bytes": (512, 1024, 64, 2056, 64, 256, False, "f32"),
}


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


def test_shapes_reach_past_32_bit_offsets():
    # the library accepts both shapes, and their largest buffers pass the 32-bit offsets
    for B, n, d, e, s, c, causal, dtype in CASES.values():
        esz = 2 if dtype == "bf16" else 4
        assert B * n * e * esz > 2**32
        code = fg.BF16 if dtype == "bf16" else fg.F32
        assert fg.workspace_size(B, n, d, e, s, c, causal, code) > 0
        if dtype == "bf16":
            assert fg.backward_workspace_size(B, n, d, e, s, c, causal, code) > 0
    B, n, _, e, *_ = CASES["bf16_2p31_elements"]
    assert B * n * e > 2**31


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(CASES))
def test_forward_past_32_bit_offsets(name):
    import torch
    B, n, d, e, s, c, causal, dtype = CASES[name]
    print(f"[gpu case] forward large offsets {name}: B={B} n={n} d={d} e={e} s={s} c={c} "
          f"causal={causal} {dtype}", flush=True)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=500, gamma_std=0.3, beta_std=0.1)
    O = fg.flash_gau_forward(*_args(inp, dtype), c, causal)
    torch.cuda.synchronize()
    sample = [0, B // 2, B - 1]
    got = O[sample].float().cpu().numpy()
    del O
    ref = oracle.flash_forward(inp.X[sample], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o,
                               c, causal)
    errs = [_rel(got[i], ref[i]) for i in range(len(sample))]
    print(f"  sequences {sample}: max rel err " + " ".join(f"{x:.3e}" for x in errs), flush=True)
    assert max(errs) <= TOL[dtype]


@pytest.mark.gpu
def test_backward_past_32_bit_offsets():
    # dO is zero on every sequence but the last, so each weight gradient is that sequence's
    # contribution alone and the oracle needs only it; the other sequences' dX must be zero
    import torch
    B, n, d, e, s, c, causal, dtype = CASES["bf16_2p31_elements"]
    print(f"[gpu case] backward large offsets: B={B} n={n} d={d} e={e} s={s} c={c} {dtype}",
          flush=True)
    inp = gen.make_inputs(B, n, d, e, s, c, causal, dtype, seed=501, gamma_std=0.3, beta_std=0.1)
    dO = gen.make_output_grad(B, n, d, dtype, seed=501)
    dO[:-1] = 0.0
    grads = fg.flash_gau_backward(*_args(inp, dtype), _dev(dO, dtype), c, causal)
    torch.cuda.synchronize()
    assert float(grads["dX"][:-1].abs().max()) == 0.0
    got = {k: (v[-1:] if k == "dX" else v).float().cpu().numpy() for k, v in grads.items()}
    del grads
    ref = oracle.flash_backward(inp.X[-1:], inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o,
                                dO[-1:], c, causal)
    errs = {k: _rel(got[k], ref[k]) for k in fg.GRAD_NAMES}
    print("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k in fg.GRAD_NAMES:
        assert errs[k] <= TOL[dtype], (k, errs[k])
