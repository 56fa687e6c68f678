"""fp64 CPU oracle for the forward and backward pass of one FLASH layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, header, table or helper with the HIP library; it takes plain NumPy arrays and
computes everything in float64.

What is computed, and where the pages define it
------------------------------------------------
Page "FLASH: Possibly the Most Interesting Efficient Transformer Design Recently"
(kexue.fm/archives/8934, English translation):

* section "Initial Power": the GLU form O = (U ⊙ V) W_o with U = SiLU(X W_u), V = SiLU(X W_v),
  W_u, W_v of shape [d, e]; Swish/SiLU on both branches.
* section "Strong Combination", equation (mix): O = (U ⊙ A V) W_o; A = I gives the GLU FFN.
* section "Weak Attention", equation (relu-att): Z = phi_z(X W_z), W_z of shape [d, s]; Q and K are
  per-dimension scale-and-offset maps of Z; relu² means relu followed by squaring; the appendix
  code normalises by 1/n² instead of the blog's 1/(ns).
* section "Mixed Chunk": split the n tokens into n/c chunks of c tokens; four scale/offset heads
  of Z_g give Q_quad, K_quad, Q_lin, K_lin; the local term is relu²(Q_quad K_quadᵀ) V inside each
  chunk (upper triangle masked for a decoder); the global term is Q_lin Σ_h K_linᵀ V_h / n, and for
  a decoder the sum runs over the earlier chunks h < g only; O_g = [U_g ⊙ (V̂_quad + V̂_lin)] W_o.

Page "大模型训练之加速篇 -attention优化" (blog.csdn.net), section 1.4 (autoregressive generation):
the RNN form of causal linear attention (a running state S_t = S_{t-1} + k_tᵀ v_t) and the cumsum
form (all outer products, then a prefix sum over tokens). Both are alternative routes to the same
global term and serve here as cross-checks.

Readings taken where the pages are silent, garbled or in conflict
------------------------------------------------------------------
* Local normalisation: relu²(Q Kᵀ / c), i.e. relu²(Q Kᵀ) / c². This is the appendix convention of
  "Weak Attention" applied per chunk (chunk = n gives the appendix's 1/n²). The blog's 1/(cs) is
  kept as the variant ``local_norm="cs"``.
* Global normalisation: 1/n (the sequence length) for both the causal and the non-causal form. The
  causal prefactor printed in "Mixed Chunk" is garbled (it is 0/0 for the first chunk); the
  "Extended Thoughts" section says the appendix divides by n. The variant ``global_norm="count"``
  divides chunk g's read-out by the number of earlier tokens (g-1)c instead (zero for g = 1).
* phi_z is SiLU, like phi_u and phi_v.
* Causal local mask: entries with key index j > query index i (inside the chunk) are zero; the
  diagonal is kept.
* Head order in gamma/beta rows: Q_quad, K_quad, Q_lin, K_lin.
* The layer has no bias, norm, residual or dropout, and by default no position encoding.
* Optional rotary position embedding (``rope_base``): the FLASH page ("Experimental Analysis")
  says every model of the paper uses RoPE but does not define it. Reading: the standard rotary
  form, interleaved pairs (x_{2k}, x_{2k+1}) of a head vector at position m rotated by the angle
  m·θ_k with θ_k = base^{-2k/s}; m is the token's index inside its sequence (0-based); it is
  applied to all four heads after their scale and offset.

Decoding, one token at a time
-----------------------------
``decode_step`` is the causal layer in the RNN form that the csdn page (section 1.4) recommends for
generation: a running linear-attention state, here advanced a whole chunk at a time (the causal
"Mixed Chunk" display reads the state of the earlier chunks only), plus the keys and values of the
current chunk for the local term. Reading: every sequence of the batch is at the same position t;
the linear state is folded after the last token of each chunk; n in the /n of the read-out is the
length the forward normalises by, passed in.

Backward pass
-------------
``flash_backward`` returns the gradients of L = Σ O ⊙ dO with respect to X, the four weight
matrices, gamma and beta. The pages motivate the chunked form by its parallel training (FLASH page,
"Mixed Chunk"; csdn page, section 1.4) but print no gradient; each step function above has a
``*_backward`` counterpart derived by the chain rule, and ``flash_backward`` runs them in reverse
order. The causal cross-chunk sum turns into an exclusive suffix sum over later chunks.

Parity status: every function below is pinned by tests that do not re-type its formula
(brute-force n×n matrices, the RNN recurrence, the chunk = n and A = I reductions, causality,
permutation equivariance, closed-form values and hand-worked fixtures; the decode step against
the rows of the causal forward and of the brute-force layer; the backward against central finite
differences of the forward and the adjoint identities of its linear steps).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "silu",
    "project",
    "scale_offset_heads",
    "local_quad",
    "chunk_states",
    "prefix_states",
    "global_linear",
    "combine",
    "flash_forward",
    "brute_force_forward",
    "forward_rows",
    "rnn_global_linear",
    "cumsum_global_linear",
    "gau_forward",
    "glu_forward",
    "quad_gau_attention",
    "rotary",
    "decode_init",
    "decode_step",
    "decode_sequence",
    "silu_grad",
    "rotary_transpose",
    "local_quad_backward",
    "global_linear_backward",
    "prefix_states_backward",
    "chunk_states_backward",
    "scale_offset_heads_backward",
    "flash_backward",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def silu(x):
    """Swish / SiLU, x · sigmoid(x) ("Initial Power": both U and V use Swish).

    Written as x / (1 + e^{-x}); for large negative x, e^{-x} overflows to inf and the quotient
    is the correct limit -0.0, so the warning is silenced.
    """
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def project(X, W_u, W_v, W_z):
    """U = SiLU(X W_u), V = SiLU(X W_v), Z = SiLU(X W_z).

    "Initial Power" (GLU with Swish on U and V) and "Weak Attention" (Z = phi_z(X W_z), W_z of
    shape [d, s]; phi_z read as SiLU). X is [..., n, d].
    """
    X = _f64(X)
    return silu(X @ _f64(W_u)), silu(X @ _f64(W_v)), silu(X @ _f64(W_z))


def scale_offset_heads(Z, gamma, beta):
    """The four per-dimension affine heads of Z ("Mixed Chunk"; "Weak Attention" likens them to
    LayerNorm's gamma and beta). gamma, beta are [4, s] in the order Q_quad, K_quad, Q_lin, K_lin.
    Returns the tuple (Q_quad, K_quad, Q_lin, K_lin), each shaped like Z."""
    Z, gamma, beta = _f64(Z), _f64(gamma), _f64(beta)
    return tuple(Z * gamma[h] + beta[h] for h in range(4))


def rotary(x, positions, base):
    """Rotary position embedding of head vectors x [..., n, s] (s even) at integer positions [n]:
    each pair (x_{2k}, x_{2k+1}) is rotated by the angle m·θ_k, θ_k = base^{-2k/s} (the standard
    rotary form; the FLASH page names RoPE in "Experimental Analysis" without defining it)."""
    x = _f64(x)
    s = x.shape[-1]
    if s % 2:
        raise ValueError("rotary embedding needs an even head size")
    k = np.arange(s // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * k / s)
    angle = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    cos, sin = np.cos(angle), np.sin(angle)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * cos - odd * sin
    out[..., 1::2] = even * sin + odd * cos
    return out


def _chunks(n, chunk):
    if chunk <= 0 or n % chunk != 0:
        raise ValueError(f"chunk {chunk} must divide n {n}")
    return n // chunk


def local_quad(Qq, Kq, V, chunk, causal, local_norm="c2", return_weights=False):
    """Quadratic attention inside each non-overlapping chunk ("Mixed Chunk", first display).

    For chunk g: W_g = relu(Q_g K_gᵀ / c)² (the adopted normalisation) or relu(Q_g K_gᵀ)² / (c s)
    (``local_norm="cs"``, the blog's own constant); when causal, entries above the diagonal are
    zeroed. V̂_quad_g = W_g V_g. Inputs are [B, n, ·]; returns V̂_quad [B, n, e] and optionally the
    weights [B, G, c, c].
    """
    Qq, Kq, V = _f64(Qq), _f64(Kq), _f64(V)
    B, n, s = Qq.shape
    G = _chunks(n, chunk)
    out = np.zeros(V.shape, dtype=np.float64)
    weights = np.zeros((B, G, chunk, chunk), dtype=np.float64)
    keep = np.tril(np.ones((chunk, chunk), dtype=bool)) if causal else np.ones((chunk, chunk), dtype=bool)
    for b in range(B):
        for g in range(G):
            rows = slice(g * chunk, (g + 1) * chunk)
            scores = Qq[b, rows] @ Kq[b, rows].T
            if local_norm == "c2":
                w = np.maximum(scores / chunk, 0.0) ** 2
            elif local_norm == "cs":
                w = np.maximum(scores, 0.0) ** 2 / (chunk * s)
            else:
                raise ValueError(local_norm)
            w = np.where(keep, w, 0.0)
            weights[b, g] = w
            out[b, rows] = w @ V[b, rows]
    return (out, weights) if return_weights else out


def chunk_states(Kl, V, chunk):
    """Per-chunk linear-attention summary T_g = K_lin_gᵀ V_g, an s×e matrix ("Mixed Chunk": the
    b(n/c)se state memory). Kl is [B, n, s], V is [B, n, e]; returns [B, G, s, e]."""
    Kl, V = _f64(Kl), _f64(V)
    B, n, s = Kl.shape
    G = _chunks(n, chunk)
    T = np.zeros((B, G, s, V.shape[-1]), dtype=np.float64)
    for g in range(G):
        rows = slice(g * chunk, (g + 1) * chunk)
        T[:, g] = np.einsum("bts,bte->bse", Kl[:, rows], V[:, rows])
    return T


def prefix_states(T, causal):
    """Cross-chunk sum of the summaries ("Mixed Chunk").

    Non-causal: every chunk sees the full sum Σ_{h=1}^{n/c} T_h. Causal: chunk g sees the exclusive
    prefix Σ_{h=1}^{g-1} T_h, so the first chunk sees zero. T is [B, G, s, e]; returns the same shape.
    """
    T = _f64(T)
    S = np.zeros_like(T)
    G = T.shape[1]
    if causal:
        run = np.zeros_like(T[:, 0])
        for g in range(G):
            S[:, g] = run
            run = run + T[:, g]
    else:
        total = T.sum(axis=1)
        for g in range(G):
            S[:, g] = total
    return S


def global_linear(Ql, S, chunk, n, global_norm="n"):
    """Global read-out V̂_lin_g = Q_lin_g S_g / n ("Mixed Chunk", second and third displays, with the
    1/n reading for both forms). ``global_norm="count"`` divides chunk g by (g-1)c instead (the
    "divide by t" remark of "Extended Thoughts", at chunk granularity); the first chunk then reads 0.
    Ql is [B, n, s], S is [B, G, s, e]; returns [B, n, e]."""
    Ql, S = _f64(Ql), _f64(S)
    B = Ql.shape[0]
    G = _chunks(n, chunk)
    out = np.zeros((B, n, S.shape[-1]), dtype=np.float64)
    for g in range(G):
        rows = slice(g * chunk, (g + 1) * chunk)
        if global_norm == "n":
            scale = 1.0 / n
        elif global_norm == "count":
            scale = 0.0 if g == 0 else 1.0 / (g * chunk)
        else:
            raise ValueError(global_norm)
        out[:, rows] = (Ql[:, rows] @ S[:, g]) * scale
    return out


def combine(U, Vq, Vl, W_o):
    """O = [U ⊙ (V̂_quad + V̂_lin)] W_o ("Mixed Chunk", last display; the gate of equation (mix))."""
    return (_f64(U) * (_f64(Vq) + _f64(Vl))) @ _f64(W_o)


def flash_forward(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal,
                  local_norm="c2", global_norm="n", return_intermediates=False, rope_base=None):
    """One FLASH layer forward in the chunked form, steps in the order of "Mixed Chunk".

    X is [B, n, d] (a 2-D [n, d] input is treated as B = 1). Returns O [B, n, d] in float64, and
    with ``return_intermediates`` also a dict of U, V, Z, the four heads, the local weights P
    [B, G, c, c], the chunk summaries T and the prefix states S [B, G, s, e], V̂_quad, V̂_lin and
    the gated product Y = U ⊙ (V̂_quad + V̂_lin). With ``rope_base`` the four heads are rotated
    (``rotary``) at their positions 0..n-1 before any use.
    """
    X = _f64(X)
    squeeze = X.ndim == 2
    if squeeze:
        X = X[None]
    n = X.shape[1]
    U, V, Z = project(X, W_u, W_v, W_z)
    Qq, Kq, Ql, Kl = scale_offset_heads(Z, gamma, beta)
    if rope_base is not None:
        pos = np.arange(n)
        Qq, Kq, Ql, Kl = (rotary(h, pos, rope_base) for h in (Qq, Kq, Ql, Kl))
    Vq, P = local_quad(Qq, Kq, V, chunk, causal, local_norm=local_norm, return_weights=True)
    T = chunk_states(Kl, V, chunk)
    S = prefix_states(T, causal)
    Vl = global_linear(Ql, S, chunk, n, global_norm=global_norm)
    Y = U * (Vq + Vl)
    O = combine(U, Vq, Vl, W_o)
    if squeeze:
        O = O[0]
    if not return_intermediates:
        return O
    inter = dict(U=U, V=V, Z=Z, Qq=Qq, Kq=Kq, Ql=Ql, Kl=Kl, P=P, T=T, S=S, Vq=Vq, Vl=Vl, Y=Y)
    return O, inter


# ---------------------------------------------------------------------------------------------
# Independent formulations used to pin the chunked oracle.
# ---------------------------------------------------------------------------------------------

def brute_force_forward(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, rope_base=None):
    """The same layer with both attention matrices materialised as full n×n arrays.

    "Mixed Chunk" says the local term is attention restricted to the block diagonal (masked to the
    lower triangle for a decoder) and that the global term equals linear attention with the full
    Q_lin, K_lin in R^{n×s}; for a decoder only keys in earlier chunks are visible. Here
    A_quad[i, j] = relu(q_i·k_j / c)² when i, j share a chunk (and j <= i if causal),
    A_lin[i, j] = ql_i·kl_j / n when chunk(j) < chunk(i) (causal) or always (non-causal), and
    O = (U ⊙ (A_quad + A_lin) V) W_o, the form of equation (mix). ``rope_base`` rotates the
    heads as in flash_forward.
    """
    X = _f64(X)
    B, n, _ = X.shape
    _chunks(n, chunk)
    U, V, Z = project(X, W_u, W_v, W_z)
    Qq, Kq, Ql, Kl = scale_offset_heads(Z, gamma, beta)
    if rope_base is not None:
        Qq, Kq, Ql, Kl = (rotary(h, np.arange(n), rope_base) for h in (Qq, Kq, Ql, Kl))
    idx = np.arange(n)
    cid = idx // chunk
    same = cid[:, None] == cid[None, :]
    if causal:
        quad_mask = same & (idx[None, :] <= idx[:, None])
        lin_mask = cid[None, :] < cid[:, None]
    else:
        quad_mask = same
        lin_mask = np.ones((n, n), dtype=bool)
    O = np.zeros((B, n, _f64(W_o).shape[1]))
    for b in range(B):
        a_quad = np.where(quad_mask, np.maximum(Qq[b] @ Kq[b].T / chunk, 0.0) ** 2, 0.0)
        a_lin = np.where(lin_mask, Ql[b] @ Kl[b].T / n, 0.0)
        O[b] = (U[b] * ((a_quad + a_lin) @ V[b])) @ _f64(W_o)
    return O


def forward_rows(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, rows, rope_base=None):
    """Selected output rows of ONE sequence, each computed on its own from the definitions, for
    sequences too long for the n×n matrices of brute_force_forward.

    X is [n, d] (one sequence); rows are token indices. Row i of chunk g = i // c gets
    local_i = Σ_j relu(qq_i·kq_j / c)² v_j over the keys j of chunk g (j <= i when causal; "Mixed
    Chunk", first display), global_i = Σ_j (ql_i·kl_j / n) v_j over the keys j of the chunks before
    g (causal) or of every chunk (non-causal; "Mixed Chunk", second and third displays, the /n
    reading), and o_i = (u_i ⊙ (local_i + global_i)) W_o (last display). U, V and the heads come
    from project and scale_offset_heads (rotated when ``rope_base`` is given). Returns
    [len(rows), d] in float64.
    """
    X = _f64(X)
    if X.ndim != 2:
        raise ValueError("forward_rows takes one sequence [n, d]")
    n = X.shape[0]
    _chunks(n, chunk)
    rows = [int(r) for r in rows]
    last = max(rows) + 1 if causal else n
    U, V, Z = project(X[:last], W_u, W_v, W_z)
    Qq, Kq, Ql, Kl = scale_offset_heads(Z, gamma, beta)
    if rope_base is not None:
        pos = np.arange(last)
        Qq, Kq, Ql, Kl = (rotary(h, pos, rope_base) for h in (Qq, Kq, Ql, Kl))
    out = np.zeros((len(rows), _f64(W_o).shape[1]))
    for k, i in enumerate(rows):
        g0 = (i // chunk) * chunk
        hi = i + 1 if causal else g0 + chunk
        w = np.maximum(Kq[g0:hi] @ Qq[i] / chunk, 0.0) ** 2
        local = w @ V[g0:hi]
        lin_keys = slice(0, g0) if causal else slice(0, n)
        glob = ((Kl[lin_keys] @ Ql[i]) / n) @ V[lin_keys]
        out[k] = (U[i] * (local + glob)) @ _f64(W_o)
    return out


def rnn_global_linear(Ql, Kl, V, chunk, n):
    """Causal global term through the token recurrence of the RNN form (csdn survey §1.4, first
    form): S_t = S_{t-1} + kl_tᵀ v_t, one token at a time. A query in chunk g reads the state as it
    stood after the last token of chunk g-1, divided by n. Returns [B, n, e]."""
    Ql, Kl, V = _f64(Ql), _f64(Kl), _f64(V)
    B, _, s = Kl.shape
    e = V.shape[-1]
    out = np.zeros((B, n, e))
    for b in range(B):
        state = np.zeros((s, e))
        state_at_chunk_start = np.zeros((s, e))
        for t in range(n):
            if t % chunk == 0:
                state_at_chunk_start = state.copy()
            out[b, t] = Ql[b, t] @ state_at_chunk_start / n
            state = state + np.outer(Kl[b, t], V[b, t])
    return out


def cumsum_global_linear(Ql, Kl, V, chunk, n):
    """Causal global term through the cumsum form (csdn survey §1.4, second form): all n outer
    products kl_tᵀ v_t as an [n, s, e] array, then a prefix sum over tokens. Chunk g reads the
    inclusive sum up to its own first token minus one. Tiny shapes only (n·s·e memory)."""
    Ql, Kl, V = _f64(Ql), _f64(Kl), _f64(V)
    B = Ql.shape[0]
    out = np.zeros((B, n, V.shape[-1]))
    for b in range(B):
        outer = Kl[b][:, :, None] * V[b][:, None, :]
        csum = np.cumsum(outer, axis=0)
        for t in range(n):
            start = (t // chunk) * chunk
            state = csum[start - 1] if start > 0 else np.zeros_like(csum[0])
            out[b, t] = Ql[b, t] @ state / n
    return out


def gau_forward(X, A, W_u, W_v, W_o):
    """Equation (mix) of "Strong Combination" with a given n×n matrix A: O = (U ⊙ A V) W_o,
    U = SiLU(X W_u), V = SiLU(X W_v). X is [n, d]."""
    X = _f64(X)
    U = silu(X @ _f64(W_u))
    V = silu(X @ _f64(W_v))
    return (U * (_f64(A) @ V)) @ _f64(W_o)


def glu_forward(X, W_u, W_v, W_o):
    """The GLU FFN of "Initial Power": O = (U ⊙ V) W_o with Swish on both branches. X is [n, d]."""
    X = _f64(X)
    return (silu(X @ _f64(W_u)) * silu(X @ _f64(W_v))) @ _f64(W_o)


def quad_gau_attention(X, W_z, gamma_q, beta_q, gamma_k, beta_k, causal):
    """The quadratic GAU's attention matrix with the appendix normalisation of "Weak Attention":
    A = relu²(Q Kᵀ) / n², Q = gamma_q ⊙ Z + beta_q, K = gamma_k ⊙ Z + beta_k, Z = SiLU(X W_z);
    the upper triangle is zeroed when causal. X is [n, d]; returns [n, n]."""
    X = _f64(X)
    n = X.shape[0]
    Z = silu(X @ _f64(W_z))
    Q = Z * _f64(gamma_q) + _f64(beta_q)
    K = Z * _f64(gamma_k) + _f64(beta_k)
    A = np.maximum(Q @ K.T, 0.0) ** 2 / float(n) ** 2
    if causal:
        A = np.tril(A)
    return A


# ---------------------------------------------------------------------------------------------
# Causal decoding in the RNN form.
# ---------------------------------------------------------------------------------------------

def decode_init(B, s, e, chunk):
    """Empty decoding state for B sequences: the linear state S [B, s, e] (Σ K_linᵀ V over the
    completed chunks) and the current chunk's K_quad [B, c, s], K_lin [B, c, s] and V [B, c, e]."""
    return dict(S=np.zeros((B, s, e)), Kq=np.zeros((B, chunk, s)), Kl=np.zeros((B, chunk, s)),
                V=np.zeros((B, chunk, e)))


def decode_step(state, x, t, n, W_u, W_v, W_z, gamma, beta, W_o, chunk,
                local_norm="c2", global_norm="n", rope_base=None):
    """Output of token t (0-based, the same position in every sequence) of the causal layer, given
    the state left by tokens 0..t-1; updates the state in place. x is [B, d]; returns o [B, d].

    Steps, in the order of "Mixed Chunk" for one token i = t mod c of chunk g = t div c: project
    and take the four heads; store k_quad, k_lin, v as row i of the chunk; local term over the keys
    0..i of the chunk (the causal mask keeps the diagonal); global term q_lin S / n with S the sum
    over the earlier chunks only (``global_norm="count"`` divides by the g·c tokens summed
    instead, 0 in the first chunk); gate and output projection. After the chunk's last token,
    S += K_lin_gᵀ V_g (the state update of the RNN form of csdn section 1.4, a chunk at a time).
    ``rope_base`` rotates the heads at position t, as flash_forward does.
    """
    x = _f64(x)
    i, g = t % chunk, t // chunk
    U, V, Z = project(x, W_u, W_v, W_z)
    Qq, Kq, Ql, Kl = scale_offset_heads(Z, gamma, beta)
    if rope_base is not None:
        Qq, Kq, Ql, Kl = (rotary(h[:, None, :], [t], rope_base)[:, 0] for h in (Qq, Kq, Ql, Kl))
    s = Z.shape[-1]
    state["Kq"][:, i] = Kq
    state["Kl"][:, i] = Kl
    state["V"][:, i] = V
    scores = np.einsum("bs,bjs->bj", Qq, state["Kq"][:, : i + 1])
    if local_norm == "c2":
        w = np.maximum(scores / chunk, 0.0) ** 2
    elif local_norm == "cs":
        w = np.maximum(scores, 0.0) ** 2 / (chunk * s)
    else:
        raise ValueError(local_norm)
    Vq = np.einsum("bj,bje->be", w, state["V"][:, : i + 1])
    if global_norm == "n":
        scale = 1.0 / n
    elif global_norm == "count":
        scale = 0.0 if g == 0 else 1.0 / (g * chunk)
    else:
        raise ValueError(global_norm)
    Vl = np.einsum("bs,bse->be", Ql, state["S"]) * scale
    o = combine(U, Vq, Vl, W_o)
    if i == chunk - 1:
        state["S"] += np.einsum("bjs,bje->bse", state["Kl"], state["V"])
    return o


def decode_sequence(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, n=None, **norms):
    """Runs decode_step over tokens 0..T-1 of X [B, T, d] from an empty state; returns the outputs
    [B, T, d] and the final state. n defaults to T."""
    X = _f64(X)
    B, T, _ = X.shape
    n = T if n is None else n
    state = decode_init(B, _f64(W_z).shape[1], _f64(W_u).shape[1], chunk)
    out = np.zeros((B, T, _f64(W_o).shape[1]))
    for t in range(T):
        out[:, t] = decode_step(state, X[:, t], t, n, W_u, W_v, W_z, gamma, beta, W_o, chunk, **norms)
    return out, state


# ---------------------------------------------------------------------------------------------
# Backward pass (training).
# ---------------------------------------------------------------------------------------------
# The FLASH page motivates the chunked form by training ("Mixed Chunk": the causal linear term
# stays parallel over chunks through a prefix sum) and the csdn page (section 1.4) by the cost of
# the serial recurrence; neither writes the gradients down. They follow from the forward steps
# above by the chain rule, taken here one step at a time in reverse order, for the scalar loss
# L = Σ O ⊙ dO (dO is the gradient of whatever loss follows the layer).


def silu_grad(x):
    """Derivative of SiLU: d/dx [x σ(x)] = σ(x) (1 + x (1 − σ(x)))."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-x))
    return sig * (1.0 + x * (1.0 - sig))


def rotary_transpose(g, positions, base):
    """Transpose of ``rotary`` at the same positions, applied to a gradient g [..., n, s]: each
    pair is rotated by −m·θ_k (a rotation's transpose is its inverse)."""
    g = _f64(g)
    s = g.shape[-1]
    k = np.arange(s // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * k / s)
    angle = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    cos, sin = np.cos(angle), np.sin(angle)
    even, odd = g[..., 0::2], g[..., 1::2]
    out = np.empty_like(g)
    out[..., 0::2] = even * cos + odd * sin
    out[..., 1::2] = -even * sin + odd * cos
    return out


def local_quad_backward(Qq, Kq, V, dVq, chunk, causal, local_norm="c2"):
    """Gradients of ``local_quad`` (V̂_quad_g = W_g V_g, W_g = relu(Q_g K_gᵀ / c)², masked when
    causal) with respect to Q_quad, K_quad and V, given dV̂_quad. With A = Q_g K_gᵀ:
    dW = dV̂ V_gᵀ, dV_g = W_gᵀ dV̂, and through relu², dA = dW ⊙ 2 relu(A/c) / c (zero where masked
    or A < 0); dQ_g = dA K_g, dK_g = dAᵀ Q_g."""
    Qq, Kq, V, dVq = _f64(Qq), _f64(Kq), _f64(V), _f64(dVq)
    B, n, s = Qq.shape
    G = _chunks(n, chunk)
    dQ, dK, dV = np.zeros_like(Qq), np.zeros_like(Kq), np.zeros_like(V)
    keep = np.tril(np.ones((chunk, chunk), dtype=bool)) if causal else np.ones((chunk, chunk), dtype=bool)
    for b in range(B):
        for g in range(G):
            rows = slice(g * chunk, (g + 1) * chunk)
            A = Qq[b, rows] @ Kq[b, rows].T
            if local_norm == "c2":
                w = np.maximum(A / chunk, 0.0) ** 2
                dw_da = 2.0 * np.maximum(A / chunk, 0.0) / chunk
            elif local_norm == "cs":
                w = np.maximum(A, 0.0) ** 2 / (chunk * s)
                dw_da = 2.0 * np.maximum(A, 0.0) / (chunk * s)
            else:
                raise ValueError(local_norm)
            w = np.where(keep, w, 0.0)
            dW = dVq[b, rows] @ V[b, rows].T
            dA = np.where(keep, dW * dw_da, 0.0)
            dQ[b, rows] = dA @ Kq[b, rows]
            dK[b, rows] = dA.T @ Qq[b, rows]
            dV[b, rows] = w.T @ dVq[b, rows]
    return dQ, dK, dV


def global_linear_backward(Ql, S, dVl, chunk, n, global_norm="n"):
    """Gradients of ``global_linear`` (V̂_lin_g = scale_g Q_lin_g S_g) with respect to Q_lin and the
    prefix states: dQ_lin_g = scale_g dV̂_lin_g S_gᵀ, dS_g = scale_g Q_lin_gᵀ dV̂_lin_g."""
    Ql, S, dVl = _f64(Ql), _f64(S), _f64(dVl)
    B = Ql.shape[0]
    G = _chunks(n, chunk)
    dQl, dS = np.zeros_like(Ql), np.zeros_like(S)
    for g in range(G):
        rows = slice(g * chunk, (g + 1) * chunk)
        if global_norm == "n":
            scale = 1.0 / n
        elif global_norm == "count":
            scale = 0.0 if g == 0 else 1.0 / (g * chunk)
        else:
            raise ValueError(global_norm)
        dQl[:, rows] = scale * (dVl[:, rows] @ np.swapaxes(S[:, g], 1, 2))
        dS[:, g] = scale * (np.swapaxes(Ql[:, rows], 1, 2) @ dVl[:, rows])
    return dQl, dS


def prefix_states_backward(dS, causal):
    """Gradient of ``prefix_states`` with respect to the chunk summaries T. Causal: S_g sums T_h over
    h < g, so dT_h sums dS_g over the later chunks g > h (an exclusive suffix sum; the last chunk's
    summary gets zero). Non-causal: every T_h receives the sum of all dS_g."""
    dS = _f64(dS)
    dT = np.zeros_like(dS)
    G = dS.shape[1]
    if causal:
        run = np.zeros_like(dS[:, 0])
        for h in range(G - 1, -1, -1):
            dT[:, h] = run
            run = run + dS[:, h]
    else:
        total = dS.sum(axis=1)
        for h in range(G):
            dT[:, h] = total
    return dT


def chunk_states_backward(Kl, V, dT, chunk):
    """Gradients of ``chunk_states`` (T_g = K_lin_gᵀ V_g): dK_lin_g = V_g dT_gᵀ, dV_g = K_lin_g dT_g."""
    Kl, V, dT = _f64(Kl), _f64(V), _f64(dT)
    n = Kl.shape[1]
    G = _chunks(n, chunk)
    dKl, dV = np.zeros_like(Kl), np.zeros_like(V)
    for g in range(G):
        rows = slice(g * chunk, (g + 1) * chunk)
        dKl[:, rows] = V[:, rows] @ np.swapaxes(dT[:, g], 1, 2)
        dV[:, rows] = Kl[:, rows] @ dT[:, g]
    return dKl, dV


def scale_offset_heads_backward(Z, gamma, dheads):
    """Gradients of ``scale_offset_heads`` (head_h = Z ⊙ γ_h + β_h) given the four head gradients:
    dZ = Σ_h γ_h ⊙ dhead_h, dγ_h = Σ_tokens Z ⊙ dhead_h, dβ_h = Σ_tokens dhead_h."""
    Z, gamma = _f64(Z), _f64(gamma)
    dZ = np.zeros_like(Z)
    dgamma = np.zeros_like(gamma)
    dbeta = np.zeros_like(gamma)
    for h in range(4):
        d = _f64(dheads[h])
        dZ += gamma[h] * d
        dgamma[h] = (Z * d).reshape(-1, Z.shape[-1]).sum(axis=0)
        dbeta[h] = d.reshape(-1, Z.shape[-1]).sum(axis=0)
    return dZ, dgamma, dbeta


def flash_backward(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, causal,
                   local_norm="c2", global_norm="n", rope_base=None):
    """Gradients of one FLASH layer (``flash_forward``, same arguments) for the loss Σ O ⊙ dO.

    Returns a dict with dX [B, n, d], dW_u, dW_v [d, e], dW_z [d, s], dgamma, dbeta [4, s] and
    dW_o [e, d], in float64. The forward steps are undone in reverse order: output projection,
    gate, the global term (read-out, cross-chunk sum, chunk summaries), the local term, the rotary
    embedding, the heads, SiLU, and the projection.
    """
    X, W_u, W_v, W_z, W_o, dO = (_f64(a) for a in (X, W_u, W_v, W_z, W_o, dO))
    squeeze = X.ndim == 2
    if squeeze:
        X, dO = X[None], dO[None]
    n = X.shape[1]
    _, it = flash_forward(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, local_norm=local_norm,
                          global_norm=global_norm, return_intermediates=True, rope_base=rope_base)
    U, V, Z = it["U"], it["V"], it["Z"]
    Hu, Hv, Hz = X @ W_u, X @ W_v, X @ W_z
    Vhat = it["Vq"] + it["Vl"]
    # O = Y W_o, Y = U ⊙ V̂
    dW_o = np.einsum("bne,bnd->ed", it["Y"], dO)
    dY = dO @ W_o.T
    dU = dY * Vhat
    dVhat = dY * U
    # the local and the global term both receive dV̂
    dQq, dKq, dV = local_quad_backward(it["Qq"], it["Kq"], V, dVhat, chunk, causal, local_norm)
    dQl, dS = global_linear_backward(it["Ql"], it["S"], dVhat, chunk, n, global_norm)
    dT = prefix_states_backward(dS, causal)
    dKl, dV_lin = chunk_states_backward(it["Kl"], V, dT, chunk)
    dV = dV + dV_lin
    dheads = [dQq, dKq, dQl, dKl]
    if rope_base is not None:
        dheads = [rotary_transpose(h, np.arange(n), rope_base) for h in dheads]
    dZ, dgamma, dbeta = scale_offset_heads_backward(Z, gamma, dheads)
    dHu, dHv, dHz = dU * silu_grad(Hu), dV * silu_grad(Hv), dZ * silu_grad(Hz)
    dX = dHu @ W_u.T + dHv @ W_v.T + dHz @ W_z.T
    grads = dict(
        dX=dX[0] if squeeze else dX,
        dW_u=np.einsum("bnd,bne->de", X, dHu),
        dW_v=np.einsum("bnd,bne->de", X, dHv),
        dW_z=np.einsum("bnd,bns->ds", X, dHz),
        dgamma=dgamma,
        dbeta=dbeta,
        dW_o=dW_o,
    )
    return grads
