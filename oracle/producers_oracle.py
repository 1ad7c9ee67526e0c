"""CPU oracle for the fused producers that emit MXFP4 activations.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library and imports nothing from the product package.

What it follows
---------------
The quadbit README ("Accuracy (real models)" and "The stack") runs its FP4
transformer block with fused RMSNorm, residual-add and SwiGLU quantizers
around the GEMMs: the kernel that produces an activation also writes it
quantized.  The pages do not print these operations, so the standard
definitions are taken, with the BF16 activation the producer would otherwise
write as the value that is quantized:

* residual add:  h = RNE_bf16(x + r)                   (exact sum, one rounding)
* RMSNorm:       y = RNE_bf16(h * gamma / sqrt(mean(h^2) + eps))
* SwiGLU:        y = RNE_bf16(silu(g) * u),  silu(g) = g / (1 + exp(-g))
* then (q, scales) = MXFP4 quantization of y, exactly as `quantize` defines it.

Here each value is computed in float64 from the BF16 inputs (the sum of
squares with math.fsum, i.e. correctly rounded) and rounded once to BF16.
"""
from __future__ import annotations

import math

import numpy as np

from .mxfp4_oracle import bf16_bits_to_f64, f64_to_bf16_bits


def add_residual(x_bits, r_bits) -> np.ndarray:
    """h = RNE_bf16(x + r) for BF16 bit patterns of equal shape."""
    x = bf16_bits_to_f64(x_bits)
    r = bf16_bits_to_f64(r_bits)
    # both are BF16 values (8 significant bits); their float64 sum rounds only when
    # their exponents differ by more than 45, far below any BF16 rounding midpoint
    return f64_to_bf16_bits(x + r)


def rmsnorm_f64(h_bits, gamma_bits, eps: float) -> np.ndarray:
    """h * gamma / sqrt(mean(h^2) + eps) per row, in float64.

    h_bits [rows, K] and gamma_bits [K] as BF16 bit patterns; eps is taken at
    its float32 value (the kernel's parameter type).
    """
    h = bf16_bits_to_f64(h_bits)
    g = bf16_bits_to_f64(gamma_bits)
    if h.ndim != 2 or g.shape != (h.shape[1],):
        raise ValueError("h must be [rows, K] and gamma [K]")
    eps64 = float(np.float32(eps))
    if not (eps64 >= 0 and math.isfinite(eps64)):
        raise ValueError("eps must be finite and non-negative")
    k = h.shape[1]
    out = np.empty_like(h)
    for i in range(h.shape[0]):
        s = math.fsum((h[i] * h[i]).tolist())       # each square is exact in float64
        inv = 1.0 / math.sqrt(s / k + eps64)
        out[i] = h[i] * inv * g
    return out


def rmsnorm_bf16(h_bits, gamma_bits, eps: float) -> np.ndarray:
    """RMSNorm output rounded once to BF16 (bit patterns)."""
    return f64_to_bf16_bits(rmsnorm_f64(h_bits, gamma_bits, eps))


def swiglu_f64(g_bits, u_bits) -> np.ndarray:
    """silu(g) * u = g * u / (1 + exp(-g)), elementwise in float64."""
    g = bf16_bits_to_f64(g_bits)
    u = bf16_bits_to_f64(u_bits)
    with np.errstate(over="ignore"):
        return g * u / (1.0 + np.exp(-g))


def swiglu_bf16(g_bits, u_bits) -> np.ndarray:
    return f64_to_bf16_bits(swiglu_f64(g_bits, u_bits))
