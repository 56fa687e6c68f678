"""Pins of the oracle's backward pass (``flash_backward`` and its step functions), on the CPU.

The pages give no gradient formulas, so nothing here re-types them. Each gradient is pinned to the
forward it differentiates: central finite differences of L = Σ O ⊙ dO through ``flash_forward``
(itself pinned by brute force, the RNN recurrence and the chunk = n and A = I reductions) on sampled
entries of every input; a directional derivative that moves every input at once; and, per step,
the adjoint identity <f(x), y> = <x, f'ᵀ(y)> for the steps that are linear in the argument. Planted
mistakes (mutants) in each step must fail at least one of these checks.
"""

import numpy as np
import pytest

import oracle
import oracle.flash_oracle as fo

INPUTS = [("X", "dX"), ("W_u", "dW_u"), ("W_v", "dW_v"), ("W_z", "dW_z"), ("gamma", "dgamma"),
          ("beta", "dbeta"), ("W_o", "dW_o")]


def _problem(B=2, n=8, d=5, e=6, s=4, seed=0):
    rng = np.random.default_rng(seed)
    p = dict(X=rng.standard_normal((B, n, d)), W_u=rng.standard_normal((d, e)) / 2,
             W_v=rng.standard_normal((d, e)) / 2, W_z=rng.standard_normal((d, s)) / 2,
             gamma=1 + 0.3 * rng.standard_normal((4, s)), beta=0.3 * rng.standard_normal((4, s)),
             W_o=rng.standard_normal((e, d)) / 2)
    dO = rng.standard_normal((B, n, d))
    return p, dO, rng


def _loss(p, dO, chunk, causal, **kw):
    return float((fo.flash_forward(**p, chunk=chunk, causal=causal, **kw) * dO).sum())


def _fd_worst(p, dO, chunk, causal, samples=4, seed=1, h=1e-5, **kw):
    grads = oracle.flash_backward(**p, dO=dO, chunk=chunk, causal=causal, **kw)
    rng = np.random.default_rng(seed)
    scale = max(np.abs(g).max() for g in grads.values())
    worst = 0.0
    for name, gname in INPUTS:
        a = p[name]
        for _ in range(samples):
            idx = tuple(int(rng.integers(0, m)) for m in a.shape)
            q = dict(p)
            q[name] = a.copy()
            q[name][idx] += h
            lp = _loss(q, dO, chunk, causal, **kw)
            q[name] = a.copy()
            q[name][idx] -= h
            lm = _loss(q, dO, chunk, causal, **kw)
            worst = max(worst, abs((lp - lm) / (2 * h) - grads[gname][idx]) / scale)
    return worst


CASES = {
    "causal_c4": dict(chunk=4, causal=True),
    "noncausal_c4": dict(chunk=4, causal=False),
    "causal_c2": dict(chunk=2, causal=True),
    "causal_c1": dict(chunk=1, causal=True),
    "causal_chunk_eq_n": dict(chunk=8, causal=True),
    "noncausal_chunk_eq_n": dict(chunk=8, causal=False),
    "causal_rope": dict(chunk=4, causal=True, rope_base=100.0),
    "noncausal_rope": dict(chunk=2, causal=False, rope_base=10.0),
    "causal_cs_count": dict(chunk=4, causal=True, local_norm="cs", global_norm="count"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gradients_match_finite_differences(name):
    p, dO, _ = _problem()
    kw = dict(CASES[name])
    assert _fd_worst(p, dO, **kw) < 1e-8


def test_directional_derivative_of_all_inputs_at_once():
    p, dO, rng = _problem(B=3, n=12, d=7, e=10, s=6, seed=4)
    for causal in (True, False):
        grads = oracle.flash_backward(**p, dO=dO, chunk=4, causal=causal, rope_base=50.0)
        direction = {k: rng.standard_normal(v.shape) for k, v in p.items()}
        h = 1e-6
        plus = {k: v + h * direction[k] for k, v in p.items()}
        minus = {k: v - h * direction[k] for k, v in p.items()}
        fd = (_loss(plus, dO, 4, causal, rope_base=50.0) - _loss(minus, dO, 4, causal, rope_base=50.0)) / (2 * h)
        an = sum(float((grads[g] * direction[k]).sum()) for k, g in INPUTS)
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_2d_input_is_one_sequence():
    p, dO, _ = _problem(B=1)
    g3 = oracle.flash_backward(**p, dO=dO, chunk=4, causal=True)
    q = dict(p, X=p["X"][0])
    g2 = oracle.flash_backward(**q, dO=dO[0], chunk=4, causal=True)
    assert np.array_equal(g2["dX"], g3["dX"][0])
    assert np.array_equal(g2["dW_u"], g3["dW_u"])


def test_causal_gradient_of_the_first_tokens_ignores_later_outputs():
    # with dO zero on the last chunk, nothing flows back into tokens that only the last chunk sees
    p, dO, _ = _problem(n=12)
    dO[:, 8:] = 0.0
    g = oracle.flash_backward(**p, dO=dO, chunk=4, causal=True)
    # tokens 8..11 influence only outputs 8..11 (their own chunk, and no later chunk exists)
    assert np.abs(g["dX"][:, 8:]).max() == 0.0


def test_single_chunk_causal_gives_no_gradient_to_the_linear_heads():
    # causal with one chunk: the global term reads an empty prefix, so Q_lin and K_lin do not matter
    p, dO, _ = _problem()
    g = oracle.flash_backward(**p, dO=dO, chunk=8, causal=True)
    assert np.abs(g["dgamma"][2:]).max() == 0.0 and np.abs(g["dbeta"][2:]).max() == 0.0
    assert np.abs(g["dgamma"][:2]).max() > 0.0


# ----------------------------------------------------------------------------- adjoint identities

def _inner(a, b):
    return float((np.asarray(a) * np.asarray(b)).sum())


def test_prefix_states_adjoint():
    rng = np.random.default_rng(5)
    T, dS = rng.standard_normal((2, 5, 3, 4)), rng.standard_normal((2, 5, 3, 4))
    for causal in (True, False):
        lhs = _inner(fo.prefix_states(T, causal), dS)
        rhs = _inner(T, fo.prefix_states_backward(dS, causal))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_chunk_states_and_global_linear_adjoints():
    rng = np.random.default_rng(6)
    B, n, s, e, c = 2, 12, 3, 5, 4
    Kl, V, Ql = rng.standard_normal((B, n, s)), rng.standard_normal((B, n, e)), rng.standard_normal((B, n, s))
    dT = rng.standard_normal((B, n // c, s, e))
    dKl, dV = fo.chunk_states_backward(Kl, V, dT, c)
    # T is bilinear in (Kl, V): the derivative in each argument is the map with the other fixed
    assert abs(_inner(fo.chunk_states(Kl, V, c), dT) - _inner(Kl, dKl)) < 1e-10
    assert abs(_inner(fo.chunk_states(Kl, V, c), dT) - _inner(V, dV)) < 1e-10
    S = rng.standard_normal((B, n // c, s, e))
    dVl = rng.standard_normal((B, n, e))
    for norm in ("n", "count"):
        dQl, dS = fo.global_linear_backward(Ql, S, dVl, c, n, norm)
        out = _inner(fo.global_linear(Ql, S, c, n, norm), dVl)
        assert abs(out - _inner(Ql, dQl)) < 1e-10 and abs(out - _inner(S, dS)) < 1e-10


def test_local_quad_is_linear_in_v():
    rng = np.random.default_rng(7)
    B, n, s, e, c = 2, 8, 3, 5, 4
    Qq, Kq, V, dVq = (rng.standard_normal(sh) for sh in ((B, n, s), (B, n, s), (B, n, e), (B, n, e)))
    for causal in (True, False):
        _, _, dV = fo.local_quad_backward(Qq, Kq, V, dVq, c, causal)
        assert abs(_inner(fo.local_quad(Qq, Kq, V, c, causal), dVq) - _inner(V, dV)) < 1e-10


def test_rotary_transpose_is_the_adjoint_and_the_inverse():
    rng = np.random.default_rng(8)
    x, g = rng.standard_normal((2, 9, 6)), rng.standard_normal((2, 9, 6))
    pos = np.arange(9) * 3
    assert abs(_inner(fo.rotary(x, pos, 30.0), g) - _inner(x, fo.rotary_transpose(g, pos, 30.0))) < 1e-12
    assert np.allclose(fo.rotary_transpose(fo.rotary(x, pos, 30.0), pos, 30.0), x, atol=1e-13)


def test_silu_grad_against_a_difference_quotient():
    x = np.linspace(-30, 30, 601)
    h = 1e-6
    fd = (fo.silu(x + h) - fo.silu(x - h)) / (2 * h)
    assert np.abs(fo.silu_grad(x) - fd).max() < 1e-8
    assert fo.silu_grad(np.array([0.0]))[0] == 0.5


# ------------------------------------------------------------------------------------- mutants

def _m_silu_grad(x):  # drops the x(1 - σ) term
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def _m_prefix_inclusive(dS, causal):  # inclusive instead of exclusive suffix
    if not causal:
        return _ORIG["prefix_states_backward"](dS, causal)
    return np.cumsum(np.asarray(dS)[:, ::-1], axis=1)[:, ::-1]


def _m_local_unmasked(Qq, Kq, V, dVq, chunk, causal, local_norm="c2"):  # forgets the causal mask
    return _ORIG["local_quad_backward"](Qq, Kq, V, dVq, chunk, False, local_norm)


def _m_local_no_two(Qq, Kq, V, dVq, chunk, causal, local_norm="c2"):  # drops the 2 of relu²
    dQ, dK, dV = _ORIG["local_quad_backward"](Qq, Kq, V, dVq, chunk, causal, local_norm)
    return dQ / 2, dK / 2, dV


def _m_local_swapped(Qq, Kq, V, dVq, chunk, causal, local_norm="c2"):  # dQ and dK exchanged
    dQ, dK, dV = _ORIG["local_quad_backward"](Qq, Kq, V, dVq, chunk, causal, local_norm)
    return dK, dQ, dV


def _m_global_no_scale(Ql, S, dVl, chunk, n, global_norm="n"):  # forgets 1/n
    dQl, dS = _ORIG["global_linear_backward"](Ql, S, dVl, chunk, n, global_norm)
    return dQl * n, dS * n


def _m_states_sign(Kl, V, dT, chunk):  # wrong sign on dK_lin
    dKl, dV = _ORIG["chunk_states_backward"](Kl, V, dT, chunk)
    return -dKl, dV


def _m_rotary_forward(g, positions, base):  # rotates the gradient forward instead of back
    return fo.rotary(g, positions, base)


def _m_heads_no_gamma(Z, gamma, dheads):  # dZ without the γ factors
    dZ, dg, db = _ORIG["scale_offset_heads_backward"](Z, gamma, dheads)
    return sum(np.asarray(h) for h in dheads), dg, db


_ORIG = {k: getattr(fo, k) for k in ("local_quad_backward", "global_linear_backward",
                                       "chunk_states_backward", "scale_offset_heads_backward",
                                       "prefix_states_backward")}

MUTANTS = {
    "silu_grad_missing_term": ("silu_grad", _m_silu_grad),
    "inclusive_suffix_sum": ("prefix_states_backward", _m_prefix_inclusive),
    "local_mask_forgotten": ("local_quad_backward", _m_local_unmasked),
    "local_factor_two_dropped": ("local_quad_backward", _m_local_no_two),
    "local_q_k_swapped": ("local_quad_backward", _m_local_swapped),
    "global_scale_forgotten": ("global_linear_backward", _m_global_no_scale),
    "states_sign": ("chunk_states_backward", _m_states_sign),
    "rotary_not_transposed": ("rotary_transpose", _m_rotary_forward),
    "heads_gamma_dropped": ("scale_offset_heads_backward", _m_heads_no_gamma),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_finite_differences_catch_the_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fo, attr, fn)
    p, dO, _ = _problem()
    worst = max(_fd_worst(p, dO, **CASES[c], samples=3)
                for c in ("causal_c4", "noncausal_c4", "causal_rope"))
    assert worst > 1e-4, f"mutant {name} not caught ({worst:.2e})"
