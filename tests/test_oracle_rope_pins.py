"""Pins of the oracle's rotary position embedding (``rotary``, ``rope_base=``), on the CPU.

The pages name RoPE without defining it; the reading (standard rotary form, interleaved pairs,
theta_k = base^(-2k/s), position = index inside the sequence, all four heads after their scale
and offset) is pinned by properties that do not re-type the rotation: a hand-worked vector
(tests/golden/rope_worked_example.txt), the identity at position 0, norm preservation, the
dependence of q·k on the position difference only, the brute-force layer, the decode step, and
the invariance of the local term when a chunk's tokens are repeated one chunk later.
"""

import os

import numpy as np
import pytest

import oracle
import oracle.flash_oracle as fo
from efficient_transformer_attention_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "rope_worked_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (t.strip() for t in line.split("=", 1))
                vals[k] = np.array([float(t) for t in v.split()])
    return vals


def test_rotary_hand_worked_vector():
    g = _golden()
    out = oracle.rotary(g["x"][None, :], [int(g["m"][0])], float(g["base"][0]))[0]
    assert np.abs(out - g["out"]).max() < 1e-14


def test_rotary_identity_at_position_zero():
    x = np.random.default_rng(0).standard_normal((3, 5, 16))
    assert np.array_equal(oracle.rotary(x, np.zeros(5, dtype=int), 10000.0), x)


def test_rotary_preserves_norms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 9, 24))
    pos = rng.integers(0, 5000, size=9)
    y = oracle.rotary(x, pos, 10000.0)
    assert _rel(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1)) < 1e-14


@pytest.mark.parametrize("shift", [1, 7, 300, 4095])
def test_rotary_scores_depend_on_position_difference_only(shift):
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((6, 32)), rng.standard_normal((6, 32))
    pq, pk = np.array([0, 3, 10, 17, 40, 99]), np.array([5, 0, 2, 33, 40, 1])
    a = (oracle.rotary(q, pq, 10000.0) * oracle.rotary(k, pk, 10000.0)).sum(-1)
    b = (oracle.rotary(q, pq + shift, 10000.0) * oracle.rotary(k, pk + shift, 10000.0)).sum(-1)
    assert _rel(b, a) < 1e-11
    c = (oracle.rotary(q, pq + shift, 10000.0) * oracle.rotary(k, pk, 10000.0)).sum(-1)
    assert _rel(c, a) > 1e-3  # a one-sided shift changes the scores


def _inp(n=16, chunk=4, causal=True, seed=3):
    return gen.make_inputs(2, n, 10, 12, 8, chunk, causal, "f32", seed=seed, gamma_std=0.3, beta_std=0.1)


def _w(inp):
    return inp.W_u, inp.W_v, inp.W_z, inp.gamma, inp.beta, inp.W_o


@pytest.mark.parametrize("causal", [True, False])
def test_rope_layer_matches_brute_force(causal):
    inp = _inp(causal=causal)
    O = oracle.flash_forward(inp.X, *_w(inp), 4, causal, rope_base=50.0)
    Bf = oracle.brute_force_forward(inp.X, *_w(inp), 4, causal, rope_base=50.0)
    assert _rel(O, Bf) < 1e-12
    assert _rel(O, oracle.flash_forward(inp.X, *_w(inp), 4, causal)) > 1e-3


def test_rope_decode_matches_forward_rows():
    inp = _inp()
    O = oracle.flash_forward(inp.X, *_w(inp), 4, True, rope_base=50.0)
    D, _ = oracle.decode_sequence(inp.X, *_w(inp), 4, rope_base=50.0)
    assert _rel(D, O) < 1e-12


def test_rope_local_term_is_invariant_to_a_whole_chunk_shift():
    # chunk 2 repeats the tokens of chunk 0: with the global head off, their local outputs agree,
    # since inside a chunk the rotated scores see only position differences
    inp = _inp(n=12, chunk=4)
    X = np.array(inp.X, copy=True)
    X[:, 8:12] = X[:, 0:4]
    gamma, beta = np.array(inp.gamma, copy=True), np.array(inp.beta, copy=True)
    gamma[2] = 0.0
    beta[2] = 0.0
    O = oracle.flash_forward(X, inp.W_u, inp.W_v, inp.W_z, gamma, beta, inp.W_o, 4, True, rope_base=50.0)
    assert _rel(O[:, 8:12], O[:, 0:4]) < 1e-12


# --------------------------------------------------------------------------------- mutants

PIN_CALLS = [
    test_rotary_hand_worked_vector,
    test_rotary_identity_at_position_zero,
    lambda: test_rotary_scores_depend_on_position_difference_only(7),
    lambda: test_rope_layer_matches_brute_force(True),
    test_rope_decode_matches_forward_rows,
    test_rope_local_term_is_invariant_to_a_whole_chunk_shift,
]

_orig_rotary = fo.rotary


def _half_split(x, positions, base):
    # pairs (k, k + s/2) instead of (2k, 2k+1)
    x = np.asarray(x, np.float64)
    s = x.shape[-1]
    perm = np.empty(s, dtype=int)
    perm[0::2], perm[1::2] = np.arange(s // 2), np.arange(s // 2) + s // 2
    y = _orig_rotary(x[..., perm], positions, base)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def _wrong_sign(x, positions, base):
    return _orig_rotary(x, -np.asarray(positions), base)


def _slow_frequencies(x, positions, base):
    return _orig_rotary(x, positions, float(base) ** 0.5)


def _one_based(x, positions, base):
    return _orig_rotary(x, np.asarray(positions) + 1, base)


def _no_rotation(x, positions, base):
    return np.asarray(x, np.float64)


MUTANTS = {
    "half_split_pairs": _half_split,
    "negative_angle": _wrong_sign,
    "sqrt_base": _slow_frequencies,
    "one_based_positions": _one_based,
    "no_rotation": _no_rotation,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_rope_pin_catches_the_mutant(name, monkeypatch):
    monkeypatch.setattr(fo, "rotary", MUTANTS[name])
    monkeypatch.setattr(oracle, "rotary", MUTANTS[name])
    failures = 0
    for call in PIN_CALLS:
        try:
            call()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught mutant {name}"


def test_keys_left_unrotated_is_caught(monkeypatch):
    # rotate only the query heads inside the forward: the chunk-shift invariance must fail
    calls = {"n": 0}

    def rotary_queries_only(x, positions, base):
        calls["n"] += 1
        # flash_forward rotates Qq, Kq, Ql, Kl in that order: leave the keys (2nd, 4th) alone
        return _orig_rotary(x, positions, base) if calls["n"] % 2 == 1 else np.asarray(x, np.float64)

    monkeypatch.setattr(fo, "rotary", rotary_queries_only)
    with pytest.raises(AssertionError):
        test_rope_local_term_is_invariant_to_a_whole_chunk_shift()
