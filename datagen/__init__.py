"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method itself (no selection, no
products, no quantisation): only random draws, dtype rounding of the draws,
and the workload shapes.  Both the CPU oracle and the GPU path receive the
arrays it returns.

Recipe (NumPy ``default_rng``, i.e. PCG64):

* activations ``X`` are Student-t with nu=4 degrees of freedom (heavy tails,
  iid features), drawn from seed ``100 + c`` for workload ``c``; the rotated
  copies used to vary the masks between bench iterations use seed
  ``300 + c + 1000*i``;
* weights are Gaussian, drawn in order from one generator seeded ``200 + c``;
* bf16 tensors are the fp32 draws rounded to nearest-even bf16 and returned
  as float32 arrays whose values are exactly representable in bf16.

The five workloads follow the layer shapes of the Q-Sparse and Turbo Sparse
pages (Llama-7B FFN 4096x11008, Mistral-7B FFN 4096x14336, a BitNet b1.58
style 4096x4096 linear, a 4096 -> 3x4096 fused QKV projection and a small
1024x1024 linear).  The pages measure quality on public suites; none of that
data is used or reproduced here: these seeded tensors stand in for it.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_round", "student_t", "normal", "k_from_fraction",
    "DRELU_BIAS", "c1_linear", "c2_relu2_ffn", "c3_i8t_linear",
    "c4_prefill_qkv", "c5_drelu_ffn", "c4_backward_grad", "MOE_BIAS", "c6_moe_drelu_ffn",
]

# Shared gate/up bias of the dReLU workload: with g ~ N(0, s^2), s ~= 1.81
# for t4 inputs and N(0, 0.02) weights, P(g + b > 0) ~= sqrt(0.1), so
# about 90% of relu(g) * relu(u) is zero (Turbo Sparse, per-layer
# zero-activation figure).
DRELU_BIAS = -0.866
# The same construction for the MoE experts' ~85% inactive neurons (Turbo
# Sparse summary, per-expert figure): P(g + b > 0) ~= sqrt(0.15).
MOE_BIAS = -0.518


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(a.shape)


def student_t(rng: np.random.Generator, shape, nu: float = 4.0, scale: float = 1.0) -> np.ndarray:
    return (scale * rng.standard_t(nu, size=shape)).astype(np.float32)


def normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.normal(0.0, std, size=shape).astype(np.float32)


def k_from_fraction(d: int, frac: str) -> int:
    """K = floor(d * p + 1/2) in exact rationals, with p given as a decimal string."""
    v = Fraction(d) * Fraction(frac) + Fraction(1, 2)
    return v.numerator // v.denominator


def _x_rng(c: int, rotation: int) -> np.random.Generator:
    return np.random.default_rng(100 + c if rotation == 0 else 300 + c + 1000 * rotation)


def c1_linear(rotation: int = 0, with_weights: bool = True) -> dict:
    """Single fp32 linear: X [8,1024] = 0.5*t4, W [1024,1024] ~ N(0, std 1/32), K = 410."""
    out = {"X": student_t(_x_rng(1, rotation), (8, 1024), scale=0.5),
           "K": k_from_fraction(1024, "0.4")}
    if with_weights:
        out["W"] = normal(np.random.default_rng(201), (1024, 1024), 1.0 / 32.0)
    return out


def c2_relu2_ffn(batch: int, rotation: int = 0, with_weights: bool = True,
                 d: int = 4096, ffn: int = 11008) -> dict:
    """Llama-7B-shaped squared-ReLU FFN decode in bf16, 40% kept at both top-K stages."""
    out = {"X": bf16_round(student_t(_x_rng(2, rotation), (batch, d))),
           "K_in": k_from_fraction(d, "0.4"), "K_mid": k_from_fraction(ffn, "0.4")}
    if with_weights:
        g = np.random.default_rng(202)
        out["W_up"] = bf16_round(normal(g, (ffn, d), 0.02))
        out["W_down"] = bf16_round(normal(g, (d, ffn), 0.02))
    return out


def c2g_relu2glu_ffn(batch: int, rotation: int = 0, with_weights: bool = True,
                     d: int = 4096, ffn: int = 11008) -> dict:
    """The same Llama-7B FFN with a gate (gated squared ReLU): C2's input and
    W_up/W_down draws unchanged, W_gate drawn after them from the same stream."""
    out = c2_relu2_ffn(batch, rotation, False, d, ffn)
    if with_weights:
        g = np.random.default_rng(202)
        out["W_up"] = bf16_round(normal(g, (ffn, d), 0.02))
        out["W_down"] = bf16_round(normal(g, (d, ffn), 0.02))
        out["W_gate"] = bf16_round(normal(g, (ffn, d), 0.02))
    return out


def c3_i8t_linear(batch: int, rotation: int = 0, with_weights: bool = True,
                  d: int = 4096, n: int = 4096) -> dict:
    """BitNet-b1.58-style linear: fp32 X = t4, fp32 source W ~ N(0, 0.02), 38.75% kept."""
    out = {"X": student_t(_x_rng(3, rotation), (batch, d)),
           "K": k_from_fraction(d, "0.3875")}
    if with_weights:
        out["W"] = normal(np.random.default_rng(203), (n, d), 0.02)
    return out


def c4_prefill_qkv(rotation: int = 0, with_weights: bool = True,
                   tokens: int = 2048, d: int = 4096, n: int = 12288) -> dict:
    """Batched prefill through a fused QKV projection in bf16, 70% kept per token."""
    out = {"X": bf16_round(student_t(_x_rng(4, rotation), (tokens, d))),
           "K": k_from_fraction(d, "0.7")}
    if with_weights:
        out["W"] = bf16_round(normal(np.random.default_rng(204), (n, d), 0.02))
    return out


def c4_backward_grad(tokens: int = 2048, n: int = 12288, rotation: int = 0) -> np.ndarray:
    """Upstream gradient dL/dY for a training step of the fused QKV projection:
    bf16 N(0, 1) of shape [tokens, n] (the loss scale is arbitrary; the
    backward is linear in it)."""
    return bf16_round(normal(np.random.default_rng(404 + 1000 * rotation), (tokens, n), 1.0))


def c5_drelu_ffn(batch: int, rotation: int = 0, with_weights: bool = True,
                 d: int = 4096, ffn: int = 14336, bias: float = DRELU_BIAS) -> dict:
    """Mistral-7B-shaped dReLU FFN decode in bf16 with shifted gate/up biases."""
    out = {"X": bf16_round(student_t(_x_rng(5, rotation), (batch, d)))}
    if with_weights:
        g = np.random.default_rng(205)
        out["W_gate"] = bf16_round(normal(g, (ffn, d), 0.02))
        out["W_up"] = bf16_round(normal(g, (ffn, d), 0.02))
        out["W_down"] = bf16_round(normal(g, (d, ffn), 0.02))
        out["b_gate"] = np.full(ffn, bias, dtype=np.float32)
        out["b_up"] = np.full(ffn, bias, dtype=np.float32)
    return out


def c6_moe_drelu_ffn(batch: int, rotation: int = 0, with_weights: bool = True, d: int = 4096,
                     ffn: int = 14336, n_experts: int = 8, bias: float = MOE_BIAS) -> dict:
    """Mixtral-47B-shaped dReLU MoE FFN decode in bf16: a router [E, d] and E
    experts with W_gate, W_up [E, ffn, d] (neuron-major) and W_down^T [E, ffn, d]
    (feature-major rows of the down projection), biases [E, ffn] = `bias`.
    Expert e's matrices come from their own generator (seed 206 + e), drawn
    in float32 to bound the host memory of the 8-expert layer."""
    out = {"X": bf16_round(student_t(_x_rng(6, rotation), (batch, d)))}
    if with_weights:
        out["W_router"] = bf16_round(normal(np.random.default_rng(216), (n_experts, d), 0.02))
        wg = np.empty((n_experts, ffn, d), dtype=np.float32)
        wu = np.empty((n_experts, ffn, d), dtype=np.float32)
        wd = np.empty((n_experts, ffn, d), dtype=np.float32)
        for e in range(n_experts):
            g = np.random.default_rng(206 + e)
            for dst in (wg, wu, wd):
                dst[e] = g.standard_normal((ffn, d), dtype=np.float32)
                dst[e] *= np.float32(0.02)
                dst[e] = bf16_round(dst[e])
        out["W_gate"], out["W_up"], out["W_down_t"] = wg, wu, wd
        out["b_gate"] = np.full((n_experts, ffn), bias, dtype=np.float32)
        out["b_up"] = np.full((n_experts, ffn), bias, dtype=np.float32)
    return out
