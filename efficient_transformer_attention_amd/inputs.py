"""Seeded synthetic inputs for one FLASH layer forward.

This module draws random numbers and rounds them to the storage precision; it holds none of the
layer's arithmetic. Tests and the benchmark hand the same arrays to the HIP library and to the fp64
oracle, so both sides see bit-identical inputs.

Recipe (shared by every workload): ``numpy.random.default_rng(seed)`` draws, in this order,
X ~ N(0, 1) [B, n, d]; W_u, W_v ~ N(0, 1/d) [d, e]; W_z ~ N(0, 1/d) [d, s]; gamma ~ N(1, gamma_std²)
[4, s]; beta ~ N(0, beta_std²) [4, s]; W_o ~ N(0, 1/e) [e, d]. X and the weights are rounded to the
storage dtype (fp32, or bf16 through fp32 with round-to-nearest-even at each step); gamma and beta
are always fp32. The rows of gamma and beta are the heads Q_quad, K_quad, Q_lin, K_lin.
"""

from __future__ import annotations

import dataclasses

import numpy as np

# name: (B, n, d, e, s, chunk, causal, dtype)
WORKLOADS = {
    "c1_noncausal_fp32_n512": (1, 512, 256, 512, 128, 128, False, "f32"),
    "c2_causal_bf16_n1024": (4, 1024, 512, 1024, 128, 256, True, "bf16"),
    "c3_causal_bf16_n4096": (8, 4096, 768, 1536, 128, 256, True, "bf16"),
    "c4_causal_bf16_n8192_c256": (2, 8192, 768, 1536, 128, 256, True, "bf16"),
    "c4_causal_bf16_n8192_c512": (2, 8192, 768, 1536, 128, 512, True, "bf16"),
    "c4_noncausal_bf16_n8192_c256": (2, 8192, 768, 1536, 128, 256, False, "bf16"),
    "c4_noncausal_bf16_n8192_c512": (2, 8192, 768, 1536, 128, 512, False, "bf16"),
    "c5_causal_bf16_n32768": (1, 32768, 1024, 2048, 128, 512, True, "bf16"),
}

HEADLINE = "c3_causal_bf16_n4096"


@dataclasses.dataclass
class LayerInputs:
    """One workload's inputs. Every array is float64 holding values exactly representable in the
    storage dtype (``dtype``: "bf16" or "f32"); gamma and beta hold fp32 values."""

    X: np.ndarray
    W_u: np.ndarray
    W_v: np.ndarray
    W_z: np.ndarray
    gamma: np.ndarray
    beta: np.ndarray
    W_o: np.ndarray
    chunk: int
    causal: bool
    dtype: str

    @property
    def shape(self):
        B, n, d = self.X.shape
        return B, n, d, self.W_u.shape[1], self.W_z.shape[1]


def round_to_f32(a: np.ndarray) -> np.ndarray:
    """Round to the nearest fp32 value (ties to even) and return it as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round to fp32, then to the nearest bf16 value (ties to even); return float64.

    bf16 keeps the top 16 bits of the fp32 pattern. Adding 0x7FFF plus the lowest kept bit and
    truncating implements round-to-nearest-even on the dropped half. Inputs here are finite."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return round_to_f32(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(B, n, d, e, s, chunk, causal, dtype, seed=0, gamma_std=0.02, beta_std=0.0,
                x_std=1.0) -> LayerInputs:
    """Draw one workload's inputs with the recipe in the module docstring."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((B, n, d)) * x_std
    W_u = rng.standard_normal((d, e)) / np.sqrt(d)
    W_v = rng.standard_normal((d, e)) / np.sqrt(d)
    W_z = rng.standard_normal((d, s)) / np.sqrt(d)
    gamma = 1.0 + gamma_std * rng.standard_normal((4, s))
    beta = beta_std * rng.standard_normal((4, s))
    W_o = rng.standard_normal((e, d)) / np.sqrt(e)
    return LayerInputs(
        X=round_to(X, dtype), W_u=round_to(W_u, dtype), W_v=round_to(W_v, dtype),
        W_z=round_to(W_z, dtype), gamma=round_to_f32(gamma), beta=round_to_f32(beta),
        W_o=round_to(W_o, dtype), chunk=int(chunk), causal=bool(causal), dtype=dtype)


def make_output_grad(B, n, d, dtype, seed=0, std=1.0) -> np.ndarray:
    """The gradient dO [B, n, d] arriving at the layer's output for a backward pass: N(0, std²),
    drawn from ``numpy.random.default_rng(seed + 1000)`` and rounded to the storage dtype."""
    rng = np.random.default_rng(seed + 1000)
    return round_to(rng.standard_normal((B, n, d)) * std, dtype)


def workload_inputs(name: str, seed: int = 0, **kw) -> LayerInputs:
    B, n, d, e, s, chunk, causal, dtype = WORKLOADS[name]
    return make_inputs(B, n, d, e, s, chunk, causal, dtype, seed=seed, **kw)


def isolate_branch(inp: LayerInputs, branch: str) -> LayerInputs:
    """Return a copy whose heads switch one branch of the token mixing off.

    ``branch="local"`` zeroes the Q_lin head (gamma[2] = beta[2] = 0), leaving only the quadratic
    in-chunk term; ``branch="linear"`` zeroes the Q_quad head (gamma[0] = beta[0] = 0), leaving only
    the cross-chunk linear term. Only the parameters change; no arithmetic of the layer is done."""
    gamma = inp.gamma.copy()
    beta = inp.beta.copy()
    row = {"local": 2, "linear": 0}[branch]
    gamma[row] = 0.0
    beta[row] = 0.0
    return dataclasses.replace(inp, gamma=gamma, beta=beta)
