"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin catches each one.

A pin that cannot fail proves nothing. Every mutant below replaces one oracle function with a
wrong variant (a dropped term, a wrong sign, index or constant, an inclusive instead of exclusive
scan, a swapped head) and reruns the pins of test_oracle_pins; at least one must fail.
"""

import numpy as np
import pytest

import oracle
import oracle.flash_oracle as fo
import test_oracle_pins as pins

PIN_CALLS = [
    lambda: pins.test_hand_worked_mixing(True),
    lambda: pins.test_hand_worked_mixing(False),
    lambda: pins.test_hand_constant_single_pair(),
    lambda: pins.test_silu_matches_tanh_identity(1.0),
    lambda: pins.test_silu_matches_tanh_identity(-3.5),
    lambda: pins.test_projection_hand_values(),
    lambda: pins.test_scale_offset_heads_hand_values(),
    lambda: pins.test_brute_force_matches_chunked(12, 4, True),
    lambda: pins.test_brute_force_matches_chunked(12, 4, False),
    lambda: pins.test_rnn_recurrence_equals_chunk_scan(12, 3),
    lambda: pins.test_chunk_equals_n_causal_is_quadratic_gau(),
    lambda: pins.test_full_layer_reduces_to_glu(),
    lambda: pins.test_causal_output_ignores_future_tokens(5),
    lambda: pins.test_noncausal_global_is_full_linear_attention(),
]


def _mutants():
    orig_prefix = fo.prefix_states
    orig_local = fo.local_quad
    orig_global = fo.global_linear
    orig_heads = fo.scale_offset_heads
    orig_combine = fo.combine
    orig_chunk_states = fo.chunk_states

    def inclusive_scan(T, causal):
        if not causal:
            return orig_prefix(T, causal)
        return np.cumsum(np.asarray(T, np.float64), axis=1)

    def scan_off_by_two(T, causal):
        S = orig_prefix(T, causal)
        if causal:
            S = np.concatenate([np.zeros_like(S[:, :1]), S[:, :-1]], axis=1)
        return S

    def blog_local_norm(Qq, Kq, V, chunk, causal, local_norm="c2", return_weights=False):
        return orig_local(Qq, Kq, V, chunk, causal, local_norm="cs", return_weights=return_weights)

    def no_causal_mask(Qq, Kq, V, chunk, causal, local_norm="c2", return_weights=False):
        return orig_local(Qq, Kq, V, chunk, False, local_norm=local_norm, return_weights=return_weights)

    def upper_mask(Qq, Kq, V, chunk, causal, local_norm="c2", return_weights=False):
        # keeps j >= i instead of j <= i
        if not causal:
            return orig_local(Qq, Kq, V, chunk, causal, local_norm, return_weights)
        flip = lambda a: a[:, ::-1]  # noqa: E731
        out = orig_local(flip(Qq), flip(Kq), flip(V), chunk, True, local_norm, return_weights)
        if return_weights:
            return flip(out[0]), out[1]
        return flip(out)

    def relu_not_squared(Qq, Kq, V, chunk, causal, local_norm="c2", return_weights=False):
        out, w = orig_local(Qq, Kq, V, chunk, causal, local_norm, True)
        w2 = np.sqrt(w)
        B, n, _ = np.shape(V)
        o2 = np.zeros_like(out)
        for g in range(n // chunk):
            r = slice(g * chunk, (g + 1) * chunk)
            o2[:, r] = np.einsum("bij,bje->bie", w2[:, g], np.asarray(V, np.float64)[:, r])
        return (o2, w2) if return_weights else o2

    def global_over_c(Ql, S, chunk, n, global_norm="n"):
        return orig_global(Ql, S, chunk, n, global_norm) * n / chunk

    def global_dropped(Ql, S, chunk, n, global_norm="n"):
        return 0.0 * orig_global(Ql, S, chunk, n, global_norm)

    def heads_swapped(Z, gamma, beta):
        qq, kq, ql, kl = orig_heads(Z, gamma, beta)
        return ql, kq, qq, kl

    def gate_sign(U, Vq, Vl, W_o):
        return orig_combine(U, Vq, -np.asarray(Vl), W_o)

    def silu_wrong_sign(x):
        x = np.asarray(x, np.float64)
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(x))

    def states_wrong_rows(Kl, V, chunk):
        # pairs K_lin of chunk g with V of the next chunk (an index slip)
        V = np.asarray(V, np.float64)
        return orig_chunk_states(Kl, np.roll(V, -chunk, axis=1), chunk)

    return {
        "inclusive_scan": ("prefix_states", inclusive_scan),
        "scan_shifted": ("prefix_states", scan_off_by_two),
        "blog_local_norm": ("local_quad", blog_local_norm),
        "no_causal_mask": ("local_quad", no_causal_mask),
        "upper_mask": ("local_quad", upper_mask),
        "relu_not_squared": ("local_quad", relu_not_squared),
        "global_over_c": ("global_linear", global_over_c),
        "global_dropped": ("global_linear", global_dropped),
        "heads_swapped": ("scale_offset_heads", heads_swapped),
        "gate_sign": ("combine", gate_sign),
        "silu_wrong_sign": ("silu", silu_wrong_sign),
        "states_wrong_rows": ("chunk_states", states_wrong_rows),
    }


MUTANTS = _mutants()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_the_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fo, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failures = 0
    for call in PIN_CALLS:
        try:
            call()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught mutant {name}"
