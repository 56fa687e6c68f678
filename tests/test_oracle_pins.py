"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test states the passage it follows. The layer's definitions are on the page "FLASH: Possibly
the Most Interesting Efficient Transformer Design Recently" (kexue.fm/archives/8934); the RNN and
cumsum forms of causal linear attention are in section 1.4 of the blog.csdn.net survey
"大模型训练之加速篇 -attention优化". All tests run on the CPU.
"""

import math
import os

import numpy as np
import pytest

import oracle
from efficient_transformer_attention_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / scale


def _small(B=2, n=16, d=12, e=10, s=6, chunk=4, causal=True, seed=0, beta_std=0.1, gamma_std=0.3):
    return gen.make_inputs(B, n, d, e, s, chunk, causal, "f32", seed=seed,
                           beta_std=beta_std, gamma_std=gamma_std)


def _args(inp, **over):
    kw = dict(X=inp.X, W_u=inp.W_u, W_v=inp.W_v, W_z=inp.W_z, gamma=inp.gamma, beta=inp.beta,
              W_o=inp.W_o, chunk=inp.chunk, causal=inp.causal)
    kw.update(over)
    return kw


# ------------------------------------------------------------------ closed forms: SiLU ("Initial Power")

@pytest.mark.parametrize("x", [0.0, 1.0, -1.0, 2.0, -3.5, 0.25, 8.0, -8.0, 30.0, -30.0])
def test_silu_matches_tanh_identity(x):
    # Swish/SiLU is x·sigmoid(x); sigmoid(x) = (1 + tanh(x/2)) / 2 is an independent route.
    want = x * (1.0 + math.tanh(x / 2.0)) / 2.0
    assert abs(oracle.silu(x) - want) <= 1e-15 * max(1.0, abs(want))


def test_silu_limits_and_reflection():
    x = np.linspace(-20, 20, 401)
    y = oracle.silu(x)
    # x·sigmoid(x) - (-x)·sigmoid(-x) = x·(sigmoid(x) + sigmoid(-x)) = x
    np.testing.assert_allclose(y - oracle.silu(-x), x, rtol=0, atol=1e-13)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(60.0) - 60.0) < 1e-20
    assert oracle.silu(-800.0) == 0.0  # overflowing exp gives the exact limit
    assert np.all(np.diff(y[y.argmin():]) > 0)  # increasing right of its minimum


def test_projection_hand_values():
    # X = [1, -1]; X W = 1 for W = [1, 0]ᵀ and [0, -1]ᵀ, X W = -2 for [-1, 1]ᵀ.
    X = np.array([[[1.0, -1.0]]])
    U, V, Z = oracle.project(X, np.array([[1.0], [0.0]]), np.array([[0.0], [-1.0]]),
                             np.array([[-1.0], [1.0]]))
    s1 = 1.0 * (1.0 + math.tanh(0.5)) / 2.0
    s_m2 = -2.0 * (1.0 + math.tanh(-1.0)) / 2.0
    assert abs(U[0, 0, 0] - s1) < 1e-15 and abs(V[0, 0, 0] - s1) < 1e-15
    assert abs(Z[0, 0, 0] - s_m2) < 1e-15


def test_scale_offset_heads_hand_values():
    Z = np.array([[[1.0, -2.0]]])
    gamma = np.array([[1.0, 2.0], [3.0, 4.0], [0.5, 0.0], [-1.0, 1.0]])
    beta = np.array([[0.0, 1.0], [0.0, 0.0], [1.0, 1.0], [2.0, -2.0]])
    heads = oracle.scale_offset_heads(Z, gamma, beta)
    want = [[1.0, -3.0], [3.0, -8.0], [1.5, 1.0], [1.0, -4.0]]
    for h, w in zip(heads, want):
        np.testing.assert_array_equal(h[0, 0], w)


# ------------------------------------------------------------------ hand-worked fixture ("Mixed Chunk")

def _load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (t.strip() for t in line.split("=", 1))
            vals[k] = np.array([float(t) for t in v.split()])
    return vals


@pytest.mark.parametrize("causal", [True, False])
def test_hand_worked_mixing(causal):
    g = _load_golden("mixing_worked_example.txt")
    n, c = int(g["n"][0]), int(g["chunk"][0])
    col = lambda a: a.reshape(1, n, 1)  # noqa: E731  [B=1, n, 1]
    Qq, Kq, Ql, Kl, V, U = (col(g[k]) for k in ("Qq", "Kq", "Ql", "Kl", "V", "U"))
    W_o = g["W_o"].reshape(1, -1)
    tag = "causal" if causal else "noncausal"
    Vq = oracle.local_quad(Qq, Kq, V, c, causal)
    T = oracle.chunk_states(Kl, V, c)
    S = oracle.prefix_states(T, causal)
    Vl = oracle.global_linear(Ql, S, c, n)
    O = oracle.combine(U, Vq, Vl, W_o)
    np.testing.assert_array_equal(Vq[0, :, 0], g[f"{tag}.Vq"])
    np.testing.assert_array_equal(S[0, :, 0, 0], g[f"{tag}.S"])
    np.testing.assert_array_equal(Vl[0, :, 0], g[f"{tag}.Vl"])
    np.testing.assert_array_equal(O[0, :, 0], g[f"{tag}.Y"])
    np.testing.assert_array_equal(O[0, :, 1], -2.0 * g[f"{tag}.Y"])


def test_hand_constant_single_pair():
    # n = c = 2, s = 1: q·k = c gives relu²(c / c) = 1; a second key with q·k = -c is cut by relu.
    Qq = np.array([[[1.0], [1.0]]])
    Kq = np.array([[[2.0], [-2.0]]])
    V = np.array([[[5.0], [7.0]]])
    Vq = oracle.local_quad(Qq, Kq, V, 2, causal=False)
    np.testing.assert_array_equal(Vq[0, :, 0], [5.0, 5.0])


# ------------------------------------------------------------------ brute force: materialised n x n attention matrices

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,chunk", [(8, 1), (8, 2), (8, 4), (8, 8), (12, 1), (12, 2), (12, 4), (12, 12),
                                     (16, 1), (16, 2), (16, 4), (16, 16)])
def test_brute_force_matches_chunked(n, chunk, causal):
    inp = _small(n=n, chunk=chunk, causal=causal, seed=n * 100 + chunk)
    O = oracle.flash_forward(**_args(inp))
    O_bf = oracle.brute_force_forward(**_args(inp))
    assert _rel(O, O_bf) <= 1e-12


def test_local_equals_mha_with_n_over_c_heads():
    # "Mixed Chunk": the local term is multi-head attention with n/c heads of length c.
    inp = _small(n=24, chunk=6, causal=True, seed=3)
    B, n, d, e, s = inp.shape
    c = inp.chunk
    U, V, Z = oracle.project(inp.X, inp.W_u, inp.W_v, inp.W_z)
    Qq, Kq, _, _ = oracle.scale_offset_heads(Z, inp.gamma, inp.beta)
    heads = lambda a: a.reshape(B, n // c, c, a.shape[-1])  # noqa: E731
    q, k, v = heads(Qq), heads(Kq), heads(V)
    att = np.einsum("bhis,bhjs->bhij", q, k)
    att = np.maximum(att / c, 0) ** 2 * np.tril(np.ones((c, c)))
    want = np.einsum("bhij,bhje->bhie", att, v).reshape(B, n, e)
    assert _rel(oracle.local_quad(Qq, Kq, V, c, True), want) <= 1e-13


# ------------------------------------------------------------------ RNN = cumsum: the token recurrence against the chunk scan

@pytest.mark.parametrize("n,chunk", [(12, 1), (12, 3), (12, 4), (16, 8), (16, 16)])
def test_rnn_recurrence_equals_chunk_scan(n, chunk):
    inp = _small(n=n, chunk=chunk, causal=True, seed=7)
    _, V, Z = oracle.project(inp.X, inp.W_u, inp.W_v, inp.W_z)
    _, _, Ql, Kl = oracle.scale_offset_heads(Z, inp.gamma, inp.beta)
    S = oracle.prefix_states(oracle.chunk_states(Kl, V, chunk), causal=True)
    scan = oracle.global_linear(Ql, S, chunk, n)
    rnn = oracle.rnn_global_linear(Ql, Kl, V, chunk, n)
    csum = oracle.cumsum_global_linear(Ql, Kl, V, chunk, n)
    assert _rel(scan, rnn) <= 1e-12
    assert _rel(scan, csum) <= 1e-12
    # the first chunk reads an empty prefix
    assert np.all(scan[:, :chunk] == 0.0)


def test_noncausal_global_is_full_linear_attention():
    # "Mixed Chunk": the non-causal global term equals linear attention with the full Q_lin, K_lin.
    inp = _small(n=20, chunk=5, causal=False, seed=11)
    _, V, Z = oracle.project(inp.X, inp.W_u, inp.W_v, inp.W_z)
    _, _, Ql, Kl = oracle.scale_offset_heads(Z, inp.gamma, inp.beta)
    S = oracle.prefix_states(oracle.chunk_states(Kl, V, 5), causal=False)
    got = oracle.global_linear(Ql, S, 5, 20)
    want = np.stack([(Ql[b] @ Kl[b].T) @ V[b] for b in range(Ql.shape[0])]) / 20
    assert _rel(got, want) <= 1e-13


# ------------------------------------------------------------------ chunk = n -> quadratic GAU (check 3)

def test_chunk_equals_n_causal_is_quadratic_gau():
    inp = _small(B=2, n=10, chunk=10, causal=True, seed=5)
    O = oracle.flash_forward(**_args(inp))
    for b in range(2):
        A = oracle.quad_gau_attention(inp.X[b], inp.W_z, inp.gamma[0], inp.beta[0],
                                      inp.gamma[1], inp.beta[1], causal=True)
        want = oracle.gau_forward(inp.X[b], A, inp.W_u, inp.W_v, inp.W_o)
        assert _rel(O[b], want) <= 1e-13


def test_chunk_equals_n_noncausal_is_quadratic_gau_without_linear_head():
    inp = gen.isolate_branch(_small(B=2, n=10, chunk=10, causal=False, seed=6), "local")
    O = oracle.flash_forward(**_args(inp))
    for b in range(2):
        A = oracle.quad_gau_attention(inp.X[b], inp.W_z, inp.gamma[0], inp.beta[0],
                                      inp.gamma[1], inp.beta[1], causal=False)
        want = oracle.gau_forward(inp.X[b], A, inp.W_u, inp.W_v, inp.W_o)
        assert _rel(O[b], want) <= 1e-13


# ------------------------------------------------------------------ A = I -> GLU FFN (check 4)

def test_identity_attention_is_glu():
    inp = _small(B=1, n=9, chunk=9, seed=8)
    got = oracle.gau_forward(inp.X[0], np.eye(9), inp.W_u, inp.W_v, inp.W_o)
    want = oracle.glu_forward(inp.X[0], inp.W_u, inp.W_v, inp.W_o)
    assert _rel(got, want) <= 1e-15


def test_full_layer_reduces_to_glu():
    # chunk 1, causal; Q_quad = K_quad = first unit vector (gamma 0, beta e1) so relu²(1/1) = 1 on the
    # diagonal; Q_lin = 0 switches the global term off. Then A = I and O = (U ⊙ V) W_o.
    inp = _small(B=2, n=7, chunk=1, causal=True, seed=9)
    s = inp.gamma.shape[1]
    gamma = inp.gamma.copy()
    beta = inp.beta.copy()
    e1 = np.zeros(s)
    e1[0] = 1.0
    gamma[0] = gamma[1] = 0.0
    beta[0] = beta[1] = e1
    gamma[2] = beta[2] = 0.0
    O = oracle.flash_forward(**_args(inp, gamma=gamma, beta=beta))
    for b in range(2):
        want = oracle.glu_forward(inp.X[b], inp.W_u, inp.W_v, inp.W_o)
        assert _rel(O[b], want) <= 1e-15


# ------------------------------------------------------------------ causality (check 5)

@pytest.mark.parametrize("t", [1, 5, 8, 13])
def test_causal_output_ignores_future_tokens(t):
    inp = _small(B=2, n=16, chunk=4, causal=True, seed=12)
    O = oracle.flash_forward(**_args(inp))
    X2 = inp.X.copy()
    X2[:, t:] = np.random.default_rng(99).standard_normal(X2[:, t:].shape) * 3
    O2 = oracle.flash_forward(**_args(inp, X=X2))
    assert _rel(O2[:, :t], O[:, :t]) <= 1e-15
    assert _rel(O2[:, t:], O[:, t:]) > 1e-3  # the future itself does change


def test_noncausal_output_sees_future_tokens():
    inp = _small(B=1, n=16, chunk=4, causal=False, seed=12)
    O = oracle.flash_forward(**_args(inp))
    X2 = inp.X.copy()
    X2[:, 12:] += 1.0
    O2 = oracle.flash_forward(**_args(inp, X=X2))
    assert _rel(O2[:, :4], O[:, :4]) > 1e-6


# ------------------------------------------------------------------ invariants

def test_permutation_equivariance_noncausal():
    inp = _small(B=1, n=16, chunk=4, causal=False, seed=13)
    O = oracle.flash_forward(**_args(inp))
    rng = np.random.default_rng(0)
    # inside every chunk
    perm = np.concatenate([g * 4 + rng.permutation(4) for g in range(4)])
    O_p = oracle.flash_forward(**_args(inp, X=inp.X[:, perm]))
    assert _rel(O_p, O[:, perm]) <= 1e-13
    # whole chunks
    order = rng.permutation(4)
    perm = np.concatenate([np.arange(g * 4, g * 4 + 4) for g in order])
    O_p = oracle.flash_forward(**_args(inp, X=inp.X[:, perm]))
    assert _rel(O_p, O[:, perm]) <= 1e-13


def test_batch_rows_are_independent():
    inp = _small(B=3, n=8, chunk=4, causal=True, seed=14)
    O = oracle.flash_forward(**_args(inp))
    O1 = oracle.flash_forward(**_args(inp, X=inp.X[1:2]))
    assert _rel(O1[0], O[1]) <= 1e-15


def test_homogeneity_of_the_heads():
    inp = _small(B=1, n=12, chunk=4, causal=True, seed=15, beta_std=0.0)
    O, it = oracle.flash_forward(**_args(inp), return_intermediates=True)
    g2 = inp.gamma.copy()
    g2[0] *= 3.0  # Q_quad scaled by 3 (beta 0): relu²(3x) = 9 relu²(x)
    _, it2 = oracle.flash_forward(**_args(inp, gamma=g2), return_intermediates=True)
    assert _rel(it2["Vq"], 9.0 * it["Vq"]) <= 1e-14
    g3 = inp.gamma.copy()
    g3[2] *= -2.0  # Q_lin scaled by -2: linear read-out scales by -2
    _, it3 = oracle.flash_forward(**_args(inp, gamma=g3), return_intermediates=True)
    assert _rel(it3["Vl"], -2.0 * it["Vl"]) <= 1e-14


def test_blog_normalisation_variant_differs_by_c_over_s():
    # relu²(x/c) versus relu²(x)/(cs): the ratio is s/c for every entry.
    inp = _small(B=1, n=16, chunk=8, s=4, seed=16)
    _, V, Z = oracle.project(inp.X, inp.W_u, inp.W_v, inp.W_z)
    Qq, Kq, _, _ = oracle.scale_offset_heads(Z, inp.gamma, inp.beta)
    a = oracle.local_quad(Qq, Kq, V, 8, True, local_norm="c2")
    b = oracle.local_quad(Qq, Kq, V, 8, True, local_norm="cs")
    assert _rel(b * 4 / 8, a) <= 1e-14


def test_count_normalisation_variant():
    # "Extended Thoughts": dividing by the number of summed tokens instead of n.
    inp = _small(B=1, n=12, chunk=4, seed=17)
    _, V, Z = oracle.project(inp.X, inp.W_u, inp.W_v, inp.W_z)
    _, _, Ql, Kl = oracle.scale_offset_heads(Z, inp.gamma, inp.beta)
    S = oracle.prefix_states(oracle.chunk_states(Kl, V, 4), True)
    by_n = oracle.global_linear(Ql, S, 4, 12)
    by_count = oracle.global_linear(Ql, S, 4, 12, global_norm="count")
    assert np.all(by_count[:, :4] == 0)
    assert _rel(by_count[:, 4:8], by_n[:, 4:8] * 12 / 4) <= 1e-14
    assert _rel(by_count[:, 8:], by_n[:, 8:] * 12 / 8) <= 1e-14


def test_branch_magnitudes_at_workload_distribution():
    # Not a pin of a printed value: records that with X ~ N(0,1), W ~ N(0, 1/fan_in), gamma ~ N(1, .02)
    # the global linear branch dominates the output (why GPU parity also tests each branch alone).
    inp = gen.make_inputs(1, 1024, 128, 256, 128, 256, True, "f32", seed=0)
    _, it = oracle.flash_forward(**_args(inp), return_intermediates=True)
    rms = lambda a: float(np.sqrt(np.mean(a ** 2)))  # noqa: E731
    assert rms(it["Vl"][:, 256:]) > 10 * rms(it["Vq"])


# ------------------------------------------------------------------ row-wise evaluation for long sequences

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,chunk,rope", [(16, 4, None), (16, 16, None), (24, 8, 100.0), (12, 1, None),
                                          (32, 32, 10.0)])
def test_forward_rows_match_chunked_and_brute_force(n, chunk, rope, causal):
    # every row, and a ragged selection, of each sequence against the chunked oracle (itself pinned
    # by brute force above) and against the materialised n x n matrices
    inp = _small(n=n, chunk=chunk, causal=causal, seed=n + chunk)
    O = oracle.flash_forward(**_args(inp), rope_base=rope)
    O_bf = oracle.brute_force_forward(**_args(inp), rope_base=rope)
    for b in range(inp.X.shape[0]):
        kw = _args(inp)
        kw["X"] = inp.X[b]
        for rows in (list(range(n)), [n - 1, 0, n // 2, 1]):
            got = oracle.forward_rows(**kw, rows=rows, rope_base=rope)
            assert _rel(got, O[b, rows]) <= 1e-12
            assert _rel(got, O_bf[b, rows]) <= 1e-12


def test_forward_rows_single_chunk_is_the_quadratic_gau():
    # chunk = n, causal: row i is (u_i ⊙ Σ_{j<=i} relu(q_i·k_j / n)² v_j) W_o (the appendix's 1/n²)
    inp = _small(B=1, n=20, chunk=20, causal=True, seed=11)
    U, V, Z = oracle.project(inp.X[0], inp.W_u, inp.W_v, inp.W_z)
    Qq, Kq, _, _ = oracle.scale_offset_heads(Z, inp.gamma, inp.beta)
    rows = [0, 7, 19]
    want = np.stack([(U[i] * sum(max(Qq[i] @ Kq[j] / 20, 0.0) ** 2 * V[j] for j in range(i + 1))) @ inp.W_o
                     for i in rows])
    kw = _args(inp)
    kw["X"] = inp.X[0]
    assert _rel(oracle.forward_rows(**kw, rows=rows), want) <= 1e-12
