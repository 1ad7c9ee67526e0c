"""Pins for the MXFP8 part of the CPU oracle (E4M3 elements, W4A8 GEMM).

The pages name MXFP8 ("fp4_quantization" page: quantizers to NVFP4/MXFP4/MXFP8
with per-block scale factors; a block-scaled matmul on MXFP8) but print no
element table, scale rule or worked example, so the pins are:

* E4M3 decode against PyTorch's float8_e4m3fn (a library routine) for all 256
  codes, and against the closed form of the grid (7 subnormals m * 2**-9, 119
  normals (1 + m/8) * 2**(E-7), largest 448, S.1111.111 NaN).
* The shared exponent over every positive finite BF16 value, from the integer
  bit fields (the oracle uses frexp).
* The element encoder against PyTorch's float32 -> float8_e4m3fn conversion
  (round to nearest even) over every value a block can present to it: every
  8-bit significand at every binade below 512.  PyTorch gives NaN above 464,
  where the MX reading saturates to 448; that range is pinned separately.
* Whole blocks worked out by hand, invariants (every nonzero block reaches the
  top binade, round trip, power-of-two and sign equivariance), and the W4A8
  GEMM against exact rational brute force.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GRID4 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_matches_torch():
    want = _torch_decode_all()
    got = O.E4M3_TABLE
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], want[~nan])
    assert np.signbit(got[0x80]) and got[0x80] == 0.0


def test_e4m3_grid_closed_form():
    mags = [0.0] + [m * 2.0 ** -9 for m in range(1, 8)]
    mags += [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)]
    assert len(mags) == 127
    assert np.array_equal(O.E4M3_MAGNITUDES, np.array(mags))
    assert O.E4M3_MAGNITUDES[-1] == 448.0 == O.E4M3_MAX
    assert np.all(np.diff(O.E4M3_MAGNITUDES) > 0)


def _floor_log2_from_bits(b: int) -> int:
    exp_field = (b >> 7) & 0xFF
    mant = b & 0x7F
    if exp_field > 0:
        return exp_field - 127
    return (mant.bit_length() - 1) - 133


def test_shared_exponent_every_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    got = O.shared_exponent_e4m3(O.bf16_bits_to_f64(bits))
    want = np.array([max(-127, min(127, _floor_log2_from_bits(int(b)) - 8)) for b in bits])
    assert np.array_equal(got, want)
    assert O.shared_exponent_e4m3(0.0) == -127
    for p in range(-118, 128):
        assert O.shared_exponent_e4m3(math.ldexp(1.0, p)) == max(-127, p - 8)


def test_encoder_matches_torch_rne_over_the_block_domain():
    # every value x * 2**-e a block can present: an 8-bit significand at any binade below 2**9
    sig = 1.0 + np.arange(128) / 128.0
    v = np.concatenate([np.ldexp(sig, j) for j in range(-24, 9)] + [np.array([0.0])])
    v = v[v < 512.0]
    got = O.encode_e4m3_magnitude(v)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inrange = v <= 464.0
    assert np.array_equal(got[inrange], t[inrange])
    # above 464 round-to-nearest-even would leave the finite range: the MX reading saturates to 448
    assert np.all(got[~inrange] == 0x7E)
    assert (~inrange).sum() > 0


def test_encoder_spot_values():
    cases = {0.0: 0x00, 2.0 ** -10: 0x00, 1.5 * 2.0 ** -9: 0x02, 7.5 * 2.0 ** -9: 0x08, 1.0: 0x38,
             1.0625: 0x38, 1.1875: 0x3A, 256.0: 0x78, 448.0: 0x7E, 460.0: 0x7E, 500.0: 0x7E, 511.0: 0x7E}
    for v, code in cases.items():
        assert int(O.encode_e4m3_magnitude(np.array([v]))[0]) == code, v
    with pytest.raises(ValueError):
        O.encode_e4m3_magnitude(np.array([512.0]))


def test_block_all_ones():
    codes, scale = O.quantize_block_values_e4m3(np.ones((1, 32)))
    # amax = 1 -> e = 0 - 8 -> byte 119; 1 * 2**8 = 256 = E4M3 (exp 15, mant 0) = 0x78
    assert int(scale[0]) == 119
    assert np.all(codes == 0x78)


def test_block_hand_worked():
    x = np.zeros((1, 32))
    x[0, 0] = 3.0          # amax: floor(log2 3) = 1 -> e = -7, byte 120; 3 * 128 = 384 = 1.5 * 2**8 -> 0x7C
    x[0, 1] = -1.0         # 128 = 2**7 -> exp 14 -> 0x70, negative -> 0xF0
    x[0, 2] = 2.0 ** -10   # 2**-3 -> exp 4 -> 0x20
    x[0, 3] = -0.0         # keeps its sign: 0x80
    x[0, 4] = 2.0 ** -17   # 2**-10 = half of the smallest subnormal, tie -> even 0
    x[0, 5] = 3.0 * 2.0 ** -17   # 1.5 * 2**-9 -> tie between subnormal codes 1 and 2 -> 2
    codes, scale = O.quantize_block_values_e4m3(x)
    assert int(scale[0]) == 120
    assert [int(c) for c in codes[0, :6]] == [0x7C, 0xF0, 0x20, 0x80, 0x00, 0x02]
    assert np.all(codes[0, 6:] == 0)


def test_zero_block():
    codes, scale = O.quantize_block_values_e4m3(np.zeros((2, 32)))
    assert np.all(codes == 0) and np.all(scale == 0)


def _random_bf16_bits(shape, rng, spread=6):
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-spread, spread + 1, size=shape[:-1] + (1,)))
    return O.f64_to_bf16_bits(x)


def test_every_nonzero_block_reaches_the_top_binade():
    rng = np.random.default_rng(1)
    bits = _random_bf16_bits((64, 256), rng)
    q, s = O.quantize_mxfp8(bits)
    top = (q.reshape(64, 8, 32) & 0x7F).max(axis=-1)
    # amax / 2**e lies in [256, 512): its code is in the exponent-15 binade (0x78..0x7E)
    assert np.all((top >= 0x78) & (top <= 0x7E))


def test_round_trip_and_equivariance():
    rng = np.random.default_rng(2)
    bits = _random_bf16_bits((16, 128), rng)
    q, s = O.quantize_mxfp8(bits)
    back = O.f64_to_bf16_bits(O.dequantize_mxfp8(q, s))
    q2, s2 = O.quantize_mxfp8(back)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    x = O.bf16_bits_to_f64(bits)
    for j in (-3, 5):
        qj, sj = O.quantize_mxfp8(O.f64_to_bf16_bits(np.ldexp(x, j)))
        assert np.array_equal(qj, q) and np.array_equal(sj.astype(int), s.astype(int) + j)
    qn, sn = O.quantize_mxfp8(O.f64_to_bf16_bits(-x))
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)


def test_dequantize_rejects_nan_codes():
    q = np.zeros((1, 32), np.uint8)
    q[0, 3] = 0x7F
    with pytest.raises(ValueError):
        O.dequantize_mxfp8(q, np.full((1, 1), 127, np.uint8))


def _frac_e4m3(code: int) -> Fraction:
    mag = code & 0x7F
    e, m = mag >> 3, mag & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


def _frac_e2m1(code: int) -> Fraction:
    v = Fraction(GRID4[code & 7]).limit_denominator()
    return -v if code & 8 else v


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 32, 0), (3, 5, 64, 1), (6, 4, 160, 2)])
def test_gemm_w4a8_tiny_exact_rational(m, n, k, seed):
    rng = np.random.default_rng(seed)
    aq = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x7E                              # no NaN codes
    # scale bytes within 124..130: every product is a multiple of
    # 2**-9 * 2**-1 * 2**-3 * 2**-3 = 2**-16 and below 448 * 6 * 2**6 < 2**18, so a
    # sum of at most 160 of them needs under 42 bits: the exact result fits
    # float64's 53 and the float64 oracle must equal it exactly
    a_s = rng.integers(124, 131, size=(m, k // 32), dtype=np.uint8)
    bq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    b_s = rng.integers(124, 131, size=(n, k // 32), dtype=np.uint8)
    got = O.gemm_w4a8_nt(aq, a_s, bq, b_s)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                a = _frac_e4m3(int(aq[i, t])) * Fraction(2) ** (int(a_s[i, t // 32]) - 127)
                byte = int(bq[j, t // 2])
                b = _frac_e2m1((byte >> 4) if t & 1 else (byte & 0xF)) * Fraction(2) ** (int(b_s[j, t // 32]) - 127)
                acc += a * b
            assert got[i, j] == float(acc), (i, j)


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 32, 3), (4, 3, 64, 4), (5, 6, 160, 5)])
def test_gemm_mxfp8_tiny_exact_rational(m, n, k, seed):
    """Both operands MXFP8, every non-NaN code, scale bytes 125..129.  Every
    product is a multiple of 2**-9 * 2**-9 * 2**-2 * 2**-2 = 2**-22 and below
    448 * 448 * 2**4 < 2**22, so in units of 2**-22 each is below 2**44 and a
    sum of at most 160 of them below 2**52: the exact result fits float64 and
    the float64 oracle must equal the rational sum exactly."""
    rng = np.random.default_rng(seed)
    aq = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
    bq = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x7E
    bq[(bq & 0x7F) == 0x7F] = 0xFE
    a_s = rng.integers(125, 130, size=(m, k // 32), dtype=np.uint8)
    b_s = rng.integers(125, 130, size=(n, k // 32), dtype=np.uint8)
    got = O.gemm_mxfp8_nt(aq, a_s, bq, b_s)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                a = _frac_e4m3(int(aq[i, t])) * Fraction(2) ** (int(a_s[i, t // 32]) - 127)
                b = _frac_e4m3(int(bq[j, t])) * Fraction(2) ** (int(b_s[j, t // 32]) - 127)
                acc += a * b
            assert got[i, j] == float(acc), (i, j)


def test_gemm_mxfp8_integer_codes_is_an_integer_matmul():
    """Scale bytes 127 and codes whose E4M3 values are the integers -16..16: the
    GEMM is an int64 matrix product, exactly (a textbook special case)."""
    rng = np.random.default_rng(11)
    ints = {int(v): c for c, v in enumerate(O.E4M3_TABLE) if np.isfinite(v) and float(v).is_integer()
            and abs(v) <= 16 and (v != 0 or c == 0)}
    m, n, k = 7, 9, 256
    ai = rng.integers(-16, 17, size=(m, k))
    bi = rng.integers(-16, 17, size=(n, k))
    aq = np.vectorize(lambda v: ints[int(v)])(ai).astype(np.uint8)
    bq = np.vectorize(lambda v: ints[int(v)])(bi).astype(np.uint8)
    ones = np.full((m, k // 32), 127, np.uint8)
    got = O.gemm_mxfp8_nt(aq, ones, bq, np.full((n, k // 32), 127, np.uint8))
    assert np.array_equal(got, (ai @ bi.T).astype(np.float64))
    # and it is not symmetric in its operands' roles: C = A . B^T, not B . A^T
    assert got.shape == (m, n)


def test_gemm_mxfp8_with_fp4_valued_b_equals_w4a8():
    """Every E2M1 value is exact in E4M3: a B operand holding the E4M3 codes of
    an MXFP4 operand's values (same scale bytes) gives the W4A8 GEMM exactly."""
    rng = np.random.default_rng(12)
    m, n, k = 6, 10, 128
    aq = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x00
    a_s = rng.integers(120, 135, size=(m, k // 32), dtype=np.uint8)
    bq4 = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    b_s = rng.integers(120, 135, size=(n, k // 32), dtype=np.uint8)
    nib = np.empty((n, k), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = bq4 & 0xF, bq4 >> 4
    to8 = {}
    for c in range(16):
        v = (-1.0 if c & 8 else 1.0) * GRID4[c & 7]
        hits = [c8 for c8 in range(256) if O.E4M3_TABLE[c8] == v and (c8 >> 7) == (c >> 3)]
        to8[c] = hits[0]
    bq8 = np.vectorize(to8.get)(nib).astype(np.uint8)
    np.testing.assert_array_equal(O.gemm_mxfp8_nt(aq, a_s, bq8, b_s), O.gemm_w4a8_nt(aq, a_s, bq4, b_s))
