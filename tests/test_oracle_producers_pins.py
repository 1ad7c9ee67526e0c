"""Pins for the fused-producer oracle (residual add, RMSNorm, SwiGLU).

* the residual add against torch's BF16 addition (computed in float32 and
  rounded once, which equals the rounding of the exact sum for BF16 inputs);
* RMSNorm against torch.nn.functional.rms_norm in float64, against closed
  forms (constant rows, a single nonzero, eps = 0 giving sign * gamma) and its
  power-of-two invariance with eps = 0;
* SwiGLU against torch.nn.functional.silu in float64 and closed forms
  (silu(0) = 0, silu(g) -> g for large g, the exact value at g = log 3);
* the BF16 outputs as the nearest-even rounding of those float64 values.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import workloads


def _bits(t: torch.Tensor):
    return workloads.bf16_bits(t.to(torch.bfloat16))


def test_residual_add_matches_torch_bf16():
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-20, 20, (64, 256), generator=g).float()))
    r = (torch.randn(64, 256, generator=g) * torch.exp2(torch.randint(-20, 20, (64, 256), generator=g).float()))
    xb, rb = x.to(torch.bfloat16), r.to(torch.bfloat16)
    assert np.array_equal(O.add_residual(_bits(xb), _bits(rb)), _bits(xb + rb))


def test_rmsnorm_matches_torch_float64():
    g = torch.Generator().manual_seed(2)
    h = torch.randn(16, 512, generator=g).to(torch.bfloat16)
    gamma = (1 + 0.1 * torch.randn(512, generator=g)).to(torch.bfloat16)
    eps = 1e-5
    ref = F.rms_norm(h.double(), (512,), weight=gamma.double(), eps=float(np.float32(eps)))
    got = O.rmsnorm_f64(_bits(h), _bits(gamma), eps)
    assert np.allclose(got, ref.numpy(), rtol=1e-14, atol=0)


def test_rmsnorm_closed_forms():
    k = 64
    gamma = torch.full((k,), 0.5).to(torch.bfloat16)
    # constant row c: y = c / sqrt(c^2 + eps) * gamma
    h = torch.full((1, k), 3.0).to(torch.bfloat16)
    y = O.rmsnorm_f64(_bits(h), _bits(gamma), 1.0)
    assert np.allclose(y, 3.0 / math.sqrt(9.0 + 1.0) * 0.5, rtol=1e-15)
    # eps = 0: sign(c) * gamma exactly
    h = torch.full((1, k), -7.0).to(torch.bfloat16)
    assert np.all(O.rmsnorm_f64(_bits(h), _bits(gamma), 0.0) == -0.5)
    # single nonzero a: y0 = a / sqrt(a^2 / K + eps) * gamma0, the rest 0
    h = torch.zeros((1, k)); h[0, 5] = 2.0
    y = O.rmsnorm_f64(_bits(h.to(torch.bfloat16)), _bits(gamma), 0.25)
    assert y[0, 5] == pytest.approx(2.0 / math.sqrt(4.0 / k + 0.25) * 0.5, rel=1e-15)
    assert np.all(np.delete(y[0], 5) == 0)


def test_rmsnorm_power_of_two_invariance():
    g = torch.Generator().manual_seed(3)
    h = torch.randn(8, 256, generator=g).to(torch.bfloat16)
    gamma = torch.randn(256, generator=g).to(torch.bfloat16)
    a = O.rmsnorm_bf16(_bits(h), _bits(gamma), 0.0)
    b = O.rmsnorm_bf16(_bits(h * 2.0 ** 17), _bits(gamma), 0.0)
    assert np.array_equal(a, b)


def test_rmsnorm_bf16_is_nearest():
    g = torch.Generator().manual_seed(4)
    h = torch.randn(4, 128, generator=g).to(torch.bfloat16)
    gamma = torch.randn(128, generator=g).to(torch.bfloat16)
    y64 = O.rmsnorm_f64(_bits(h), _bits(gamma), 1e-6)
    yb = O.bf16_bits_to_f64(O.rmsnorm_bf16(_bits(h), _bits(gamma), 1e-6))
    # within half a BF16 ulp (2^-8 relative spacing at the value's binade) of the float64 value
    ulp = np.ldexp(1.0, np.frexp(np.abs(y64))[1] - 8)
    assert np.all(np.abs(yb - y64) <= ulp / 2)


def test_swiglu_matches_torch_float64_and_closed_forms():
    g = torch.Generator().manual_seed(5)
    gate = (torch.randn(32, 256, generator=g) * 4).to(torch.bfloat16)
    up = torch.randn(32, 256, generator=g).to(torch.bfloat16)
    ref = F.silu(gate.double()) * up.double()
    assert np.allclose(O.swiglu_f64(_bits(gate), _bits(up)), ref.numpy(), rtol=1e-14, atol=1e-300)
    z = torch.zeros(1, 4).to(torch.bfloat16)
    one = torch.ones(1, 4).to(torch.bfloat16)
    assert np.all(O.swiglu_f64(_bits(z), _bits(one)) == 0)
    big = torch.full((1, 4), 64.0).to(torch.bfloat16)
    assert np.all(np.abs(O.swiglu_f64(_bits(big), _bits(one)) - 64.0) < 1e-24)   # silu(g) -> g
    # g = 2: silu = 2 / (1 + e^-2)
    two = torch.full((1, 1), 2.0).to(torch.bfloat16)
    assert O.swiglu_f64(_bits(two), _bits(one[:, :1]))[0, 0] == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    # very negative gates underflow to signed zero, never NaN
    neg = torch.full((1, 2), -1000.0).to(torch.bfloat16)
    out = O.swiglu_f64(_bits(neg), _bits(one[:, :2]))
    assert np.all(out == 0) and np.all(np.signbit(out))
