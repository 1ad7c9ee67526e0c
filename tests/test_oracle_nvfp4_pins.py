"""Pins for the NVFP4 oracle (two-level: per-16 UE4M3 scale, per-row fp32 global scale).

* hand-worked rows whose bytes are written out below (uniform block, a block at
  half the row maximum, a zero row, signed zeros);
* the UE4M3 scale rounding re-derived a second way (integer quantum and rint,
  instead of the brute-force nearest search the oracle uses) over every block
  of random rows;
* invariants: power-of-two scaling of a row leaves codes and scale bytes
  unchanged and scales gs exactly; negation flips exactly the sign bits; the
  largest block of a row gets scale 448; every element's error is within half
  a grid step of its block (or the saturation distance);
* the GEMM against exact rational arithmetic on tiny shapes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads


def _bits(t):
    return workloads.bf16_bits(t.to(torch.bfloat16))


def test_uniform_block_hand_worked():
    x = torch.ones(1, 32)
    q, s, gs = O.quantize_nvfp4(_bits(x))
    assert gs[0] == np.float32(1.0) / np.float32(2688.0)
    assert s.tolist() == [[0x7E, 0x7E]]          # 448 = 1.75 * 2^8: exponent field 15, mantissa 6
    assert np.all(q == 0x77)                    # every element is code 7 (6.0)
    assert np.allclose(O.dequantize_nvfp4(q, s, gs), 1.0, rtol=2 ** -22)


def test_half_amplitude_block_hand_worked():
    x = torch.cat([torch.ones(1, 16), -0.5 * torch.ones(1, 16)], dim=1)
    q, s, gs = O.quantize_nvfp4(_bits(x))
    assert s.tolist() == [[0x7E, 0x76]]          # 448, then 224 = 1.75 * 2^7
    assert np.all(q[0, :8] == 0x77) and np.all(q[0, 8:] == 0xFF)   # -6.0 is code 15


def test_zero_row_and_signed_zero():
    x = torch.zeros(2, 32)
    x[1, 3] = -0.0
    q, s, gs = O.quantize_nvfp4(_bits(x))
    assert np.all(gs == 1.0) and np.all(s == 0)
    assert q[0].tolist() == [0] * 16
    assert q[1, 1] == 0x80 and np.sum(q[1]) == 0x80          # element 3 (high nibble of byte 1) keeps its sign


def _e4m3_rne_by_quantum(t):
    """Nearest UE4M3 value of t >= 0 (ties to even), saturated at 448: q = 2^max(floor(log2 t) - 3, -9)."""
    out = np.zeros_like(t, dtype=np.float64)
    nz = t > 0
    e = np.floor(np.log2(t[nz]))
    qexp = np.maximum(e - 3, -9)
    n = np.rint(t[nz] / np.exp2(qexp))                       # rint rounds half to even
    out[nz] = np.minimum(n * np.exp2(qexp), 448.0)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_scale_rounding_rederived(seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-30, 30, (64, 16, 1), generator=g).float()).repeat_interleave(16, 1).view(64, 256)
    xb = _bits(x)
    q, s, gs = O.quantize_nvfp4(xb)
    xf = O.bf16_bits_to_f64(xb).astype(np.float32).reshape(64, 16, 16)
    amax_b = np.abs(xf).max(axis=2)
    t = (amax_b / (np.float32(6) * gs)[:, None].astype(np.float32)).astype(np.float32)
    want = _e4m3_rne_by_quantum(t.astype(np.float64))
    assert np.array_equal(O.E4M3_TABLE[s], want)


def test_power_of_two_and_sign_equivariance():
    g = torch.Generator().manual_seed(4)
    x = torch.randn(16, 128, generator=g).to(torch.bfloat16)
    q, s, gs = O.quantize_nvfp4(_bits(x))
    q2, s2, gs2 = O.quantize_nvfp4(_bits(x * 2.0 ** 20))
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(gs2, gs * np.float32(2.0 ** 20))
    q3, s3, gs3 = O.quantize_nvfp4(_bits(-x))
    assert np.array_equal(q3, q ^ 0x88) and np.array_equal(s3, s) and np.array_equal(gs3, gs)


def test_largest_block_scale_and_error_bound():
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(32, 512, generator=g) * 3).to(torch.bfloat16)
    xb = _bits(x)
    q, s, gs = O.quantize_nvfp4(xb)
    xf = O.bf16_bits_to_f64(xb).reshape(32, 32, 16)
    amax_b = np.abs(xf).max(axis=2)
    top = np.argmax(amax_b, axis=1)
    assert np.all(s[np.arange(32), top] == 0x7E)                 # the row maximum's block scale is 448
    xh = O.dequantize_nvfp4(q, s, gs).reshape(32, 32, 16)
    d = (O.E4M3_TABLE[s] * gs[:, None])[:, :, None]
    v = np.abs(xf) / d
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    bound = np.where(v <= 6, step / 2, v - 6 + 0.0) * d * (1 + 2 ** -20)
    assert np.all(np.abs(xh - xf) <= bound + 1e-300)


def test_gemm_exact_rational_tiny():
    g = torch.Generator().manual_seed(6)
    a = (torch.randn(3, 64, generator=g) * 4).to(torch.bfloat16)
    b = torch.randn(5, 64, generator=g).to(torch.bfloat16)
    aq, as_, ag = O.quantize_nvfp4(_bits(a))
    bq, bs, bg = O.quantize_nvfp4(_bits(b))
    c = O.gemm_nvfp4_nt(aq, as_, ag, bq, bs, bg)
    da = O.dequantize_nvfp4(aq, as_, ag)
    db = O.dequantize_nvfp4(bq, bs, bg)
    for i in range(3):
        for j in range(5):
            exact = sum(Fraction(float(da[i, k])) * Fraction(float(db[j, k])) for k in range(64))
            assert abs(Fraction(float(c[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 300)
    # each dequantized value is e2m1 * ue4m3 * gs exactly (no rounding in float64)
    codes = O.unpack_codes(aq).reshape(3, 4, 16)
    recon = O.E2M1_TABLE[codes] * O.E4M3_TABLE[as_][..., None] * ag.astype(np.float64)[:, None, None]
    assert np.array_equal(recon.reshape(3, 64), da)
