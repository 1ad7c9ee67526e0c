"""Pins for the CPU oracle: each check ties it to something other than itself.

The pages print no worked numeric example for MXFP4, so the pins are closed
forms of the format, exhaustive alternative derivations, brute force in exact
rational arithmetic and library routines:

* E2M1 decode against the literal value grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}
  and its negatives (the E2M1 element format named on the DeepGEMM page,
  Summary: "packed E2M1").
* E8M0 decode against math.ldexp.
* The shared exponent over every positive finite BF16 value, derived a second
  way from the integer bit fields (the oracle uses frexp).
* The element encoder (brute-force nearest with ties to the even code) against
  the threshold-count form of round-to-nearest-even with saturation, over every
  finite BF16 magnitude and every exponent the scale can take.
* Whole blocks whose bytes are worked out by hand below (nibble order, scale
  byte, zero block, signed zero, saturation, ties).
* Invariants: every nonzero block hits the top two magnitudes, quantize
  after dequantize is the identity on quantized data, power-of-two and sign
  equivariance, row independence.
* GEMM: exact rational brute force on tiny shapes; the all-scales-127 case
  as an integer matmul; the float32 variant within the float32 error bound.
* BF16 output rounding against torch's float32 -> bfloat16 conversion.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ----------------------------------------------------------------- formats

def test_e2m1_decode_matches_value_grid():
    assert list(O.E2M1_TABLE[:8]) == GRID
    assert list(O.E2M1_TABLE[8:]) == [-g for g in GRID]
    # code 8 is negative zero
    assert O.E2M1_TABLE[8] == 0.0 and math.copysign(1.0, O.E2M1_TABLE[8]) == -1.0
    for c in range(16):
        assert O.e2m1_value(c) == O.E2M1_TABLE[c]


def test_e8m0_decode():
    b = np.arange(255)
    got = O.e8m0_value(b)
    for i in range(255):
        assert got[i] == math.ldexp(1.0, i - 127)
    with pytest.raises(ValueError):
        O.e8m0_value(255)


def _floor_log2_from_bits(bits: int) -> int:
    exp_field = bits >> 7
    mant = bits & 0x7F
    if exp_field > 0:
        return exp_field - 127
    return (mant.bit_length() - 1) - 133


def test_shared_exponent_every_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)          # positive, finite, nonzero
    vals = O.bf16_bits_to_f64(bits)
    got = O.shared_exponent(vals)
    want = np.array([max(-127, min(127, _floor_log2_from_bits(int(b)) - 2)) for b in bits])
    assert np.array_equal(got, want)
    assert O.shared_exponent(0.0) == -127
    # 2**p gives p - 2, the next BF16 value below 2**p gives p - 3
    for p in range(-120, 127):
        assert O.shared_exponent(math.ldexp(1.0, p)) == max(-127, p - 2)
        below = math.ldexp(255.0, p - 8)                  # (2 - 2**-7) * 2**(p-1)
        assert O.shared_exponent(below) == max(-127, p - 3)


def _threshold_code(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto the E2M1 grid with saturation, as a sum of comparisons.

    Midpoints of the grid are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; a tie goes
    up exactly when the upper neighbour has the even code (0.75, 1.75, 3.5).
    """
    return ((v > 0.25).astype(np.int64) + (v >= 0.75) + (v > 1.25) + (v >= 1.75)
            + (v > 2.5) + (v >= 3.5) + (v > 5.0))


def test_encoder_every_bf16_magnitude_every_exponent():
    mags = O.bf16_bits_to_f64(np.arange(0, 0x7F80, dtype=np.uint16))   # all finite magnitudes
    for e in range(-127, 126):
        v = np.ldexp(mags, -e)
        v = v[v < 8.0]          # a block with exponent e has every |x| / 2**e below 8
        got = O.encode_e2m1_magnitude(v)
        want = _threshold_code(v)
        assert np.array_equal(got, want), f"exponent {e}"


def test_encoder_rejects_values_outside_block_range():
    with pytest.raises(ValueError):
        O.encode_e2m1_magnitude(np.array([8.0]))


def test_encoder_spot_values():
    for e in (-127, -3, 0, 5, 120):
        s = math.ldexp(1.0, e)
        v = np.array([5 * s, 7.5 * s, 0.25 * s, 0.75 * s, 1.25 * s, 1.75 * s, 2.5 * s, 3.5 * s, 6 * s, 7.99 * s]) / s
        assert list(O.encode_e2m1_magnitude(v)) == [6, 7, 0, 2, 2, 4, 4, 6, 7, 7]


# ------------------------------------------------------- hand-worked blocks

def _bf16(vals):
    return O.f64_to_bf16_bits(np.asarray(vals, dtype=np.float64))


def test_block_all_ones():
    # amax 1 -> floor(log2 1) - 2 = -2 -> scale byte 125; 1 / 2**-2 = 4 -> code 6
    q, s = O.quantize(_bf16(np.ones((1, 32))))
    assert s.tolist() == [[125]]
    assert q.tolist() == [[0x66] * 16]


def test_block_nibble_order_and_codes():
    # amax 4 -> e = 0 -> byte 127.  Elements (scaled by 2**0):
    #  x0 = 4 -> code 6, x1 = 2 -> code 4        byte0 = 0x6 | 0x4 << 4 = 0x46
    #  x2 = -1.5 -> 0x8|3 = 0xB, x3 = 0.25 -> 0 (tie to even) byte1 = 0x0B
    #  x4 = 0.75 -> 2 (tie to even 1.0), x5 = -3.5 -> 0x8|6 = 0xE   byte2 = 0xE2
    #  x6 = 2.5 -> 4 (tie to 2.0), x7 = -0.0 -> 0x8             byte3 = 0x84
    #  remaining 24 elements 0 -> 0x00
    x = np.zeros((1, 32))
    x[0, :8] = [4.0, 2.0, -1.5, 0.25, 0.75, -3.5, 2.5, -0.0]
    q, s = O.quantize(_bf16(x))
    assert s.tolist() == [[127]]
    assert q[0, :4].tolist() == [0x46, 0x0B, 0xE2, 0x84]
    assert q[0, 4:].tolist() == [0] * 12


def test_block_saturation():
    # amax 7.5 -> floor(log2 7.5) = 2 -> e = 0; 7.5 > 6 saturates to code 7,
    # 5 ties between 4 and 6 -> even code 6 (value 4)
    x = np.zeros((1, 32))
    x[0, 0] = 7.5
    x[0, 1] = -5.0
    q, s = O.quantize(_bf16(x))
    assert s.tolist() == [[127]]
    assert q[0, 0] == (0x7 | (0xE << 4))


def test_zero_and_negative_zero_blocks():
    x = np.zeros((2, 32))
    x[1] = -0.0
    q, s = O.quantize(_bf16(x))
    assert s.tolist() == [[0], [0]]
    assert q[0].tolist() == [0] * 16
    assert q[1].tolist() == [0x88] * 16


def test_subnormal_block_keeps_small_codes():
    # amax = 2**-133 (smallest BF16 subnormal) -> e = -135 clamps to -127;
    # 2**-133 / 2**-127 = 2**-6 -> code 0.  amax = 2**-126 -> e = -128 -> -127;
    # 2**-126 / 2**-127 = 2 -> code 4.
    x = np.zeros((2, 32))
    x[0, 0] = math.ldexp(1.0, -133)
    x[1, 0] = math.ldexp(1.0, -126)
    x[1, 1] = -math.ldexp(1.0, -128)     # 0.5 -> code 1, negative
    q, s = O.quantize(_bf16(x))
    assert s.tolist() == [[0], [0]]
    assert q[0, 0] == 0x00
    assert q[1, 0] == (0x4 | (0x9 << 4))


def test_largest_bf16_block():
    big = float(np.ldexp(255.0, 120))          # largest finite BF16
    x = np.zeros((1, 32))
    x[0, 0] = big
    q, s = O.quantize(_bf16(x))
    # floor(log2) = 127 -> e = 125 -> byte 252; big / 2**125 = 7.97 -> saturates to code 7
    assert s.tolist() == [[252]]
    assert q[0, 0] & 0xF == 7


# -------------------------------------------------------------- invariants

def _random_bf16(rows, k, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k))
    if spread:
        x *= np.ldexp(1.0, rng.integers(-30, 30, size=(rows, k // 32, 1))).repeat(32, axis=2).reshape(rows, k)
        x[:, rng.integers(0, k, size=max(1, k // 100))] *= 20
    return O.f64_to_bf16_bits(x)


def test_every_nonzero_block_hits_top_magnitudes():
    xb = _random_bf16(64, 1024, 1)
    q, s = O.quantize(xb)
    codes = O.unpack_codes(q).reshape(64, 32, 32) & 7
    assert np.all(codes.max(axis=-1) >= 6)


def test_quantize_dequantize_round_trip_is_identity():
    xb = _random_bf16(32, 512, 2)
    xb[0, :32] = 0x8000            # a block of -0
    xb[1, 32:64] = 0               # a block of +0
    q, s = O.quantize(xb)
    deq = O.dequantize(q, s)
    back = torch.from_numpy(deq).to(torch.bfloat16)
    assert torch.equal(back.to(torch.float64), torch.from_numpy(deq)), "dequantized values are BF16-exact"
    xb2 = back.view(torch.int16).numpy().view(np.uint16)
    q2, s2 = O.quantize(xb2)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_power_of_two_and_sign_equivariance():
    xb = _random_bf16(16, 256, 3, spread=False)        # scale bytes far from the clamps
    q, s = O.quantize(xb)
    x = O.bf16_bits_to_f64(xb)
    for j in (-5, 1, 7):
        q2, s2 = O.quantize(O.f64_to_bf16_bits(np.ldexp(x, j)))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2.astype(int), s.astype(int) + j)
    qn, sn = O.quantize(xb ^ np.uint16(0x8000))
    assert np.array_equal(qn, q ^ np.uint8(0x88)) and np.array_equal(sn, s)


def test_row_independence():
    xb = _random_bf16(40, 256, 4)
    q, s = O.quantize(xb)
    idx = np.random.default_rng(5).permutation(40)[:17]
    qg, sg = O.quantize(xb[idx])
    assert np.array_equal(qg, q[idx]) and np.array_equal(sg, s[idx])


def test_dequantize_error_bound():
    # |x - x_hat| <= 2**(e+1): the widest grid gap (4..6) gives at most 1 * 2**e,
    # saturation (6, 8) at most 2 * 2**e.
    xb = _random_bf16(64, 512, 6)
    q, s = O.quantize(xb)
    x = O.bf16_bits_to_f64(xb)
    err = np.abs(x - O.dequantize(q, s)).reshape(64, 16, 32)
    bound = np.ldexp(1.0, s.astype(np.int32) - 127 + 1)[..., None]
    assert np.all(err <= bound)


# ------------------------------------------------------------------- GEMMs

def _random_operand(rows, k, rng, lo=120, hi=134):
    q = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    s = rng.integers(lo, hi + 1, size=(rows, k // 32), dtype=np.uint8)
    return q, s


def _fraction_decode(q, s):
    rows, half = q.shape
    out = []
    for r in range(rows):
        row = []
        for j in range(half * 2):
            byte = int(q[r, j // 2])
            code = (byte >> 4) if (j & 1) else (byte & 0xF)
            mag = Fraction(GRID[code & 7]).limit_denominator()
            val = -mag if code & 8 else mag
            row.append(val * Fraction(2) ** (int(s[r, j // 32]) - 127))
        out.append(row)
    return out


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 32, 0), (3, 5, 64, 1), (8, 8, 256, 2), (7, 2, 160, 3)])
def test_gemm_tiny_exact_rational(m, n, k, seed):
    rng = np.random.default_rng(seed)
    aq, as_ = _random_operand(m, k, rng)
    bq, bs = _random_operand(n, k, rng)
    got = O.gemm_nt(aq, as_, bq, bs)
    A = _fraction_decode(aq, as_)
    B = _fraction_decode(bq, bs)
    for i in range(m):
        for j in range(n):
            exact = sum((A[i][t] * B[j][t] for t in range(k)), Fraction(0))
            assert got[i, j] == float(exact), (i, j)


def test_gemm_unit_scales_is_integer_matmul():
    rng = np.random.default_rng(7)
    m, n, k = 33, 17, 512
    aq = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    ones_a = np.full((m, k // 32), 127, np.uint8)
    ones_b = np.full((n, k // 32), 127, np.uint8)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)    # 2 * grid magnitude

    def ints(q):
        lo = (q & 0xF).astype(np.int64)
        hi = (q >> 4).astype(np.int64)
        codes = np.empty((q.shape[0], q.shape[1] * 2), np.int64)
        codes[:, 0::2] = lo
        codes[:, 1::2] = hi
        return np.where(codes & 8, -1, 1) * twice[codes & 7]

    want = (ints(aq) @ ints(bq).T).astype(np.float64) / 4.0
    got = O.gemm_nt(aq, ones_a, bq, ones_b)
    assert np.array_equal(got, want)


def test_gemm_f32_within_float32_bound():
    rng = np.random.default_rng(8)
    m, n, k = 16, 24, 2048
    aq, as_ = _random_operand(m, k, rng, 110, 140)
    bq, bs = _random_operand(n, k, rng, 110, 140)
    c64 = O.gemm_nt(aq, as_, bq, bs)
    c32 = O.gemm_nt_f32(aq, as_, bq, bs)
    absprod = np.abs(O.dequantize(aq, as_)) @ np.abs(O.dequantize(bq, bs)).T
    bound = k * np.finfo(np.float32).eps * absprod
    assert np.all(np.abs(c32 - c64) <= bound)
    assert c32.dtype == np.float32


def test_gemm_f32_accumulates_in_float32():
    """The fp32 reference really accumulates in float32, not in float64 then cast.
    Every product is 0.5 * 2**-74 times 0.5 * 2**-74 = 2**-150: exactly half the
    smallest float32 subnormal, which rounds (ties to even) to zero.  So in any
    float32 order, with or without fused multiply-add, every partial sum stays
    zero, while the exact sum of 64 such products is 2**-144, a float32
    subnormal that a float64 accumulation followed by a cast would keep."""
    k = 64
    code_half = 0x1                                  # E2M1 code of 0.5
    q = np.full((1, k // 2), code_half | (code_half << 4), np.uint8)
    s = np.full((1, k // 32), 127 - 74, np.uint8)    # 2**-74
    c64 = O.gemm_nt(q, s, q, s)
    c32 = O.gemm_nt_f32(q, s, q, s)
    assert c64[0, 0] == 2.0 ** -144
    assert np.float32(c64[0, 0]) == np.float32(2.0 ** -144) != 0
    assert c32[0, 0] == 0.0


def test_grouped_gemm_tiny_exact_rational():
    rng = np.random.default_rng(9)
    k, n = 64, 3
    offsets = np.array([0, 2, 2, 5, 6])                 # group 1 empty
    total = offsets[-1]
    aq, as_ = _random_operand(total, k, rng)
    bq = rng.integers(0, 256, size=(4, n, k // 2), dtype=np.uint8)
    bs = rng.integers(120, 135, size=(4, n, k // 32), dtype=np.uint8)
    got = O.grouped_gemm_nt(aq, as_, bq, bs, offsets)
    A = _fraction_decode(aq, as_)
    for g in range(4):
        B = _fraction_decode(bq[g], bs[g])
        for r in range(offsets[g], offsets[g + 1]):
            for j in range(n):
                exact = sum((A[r][t] * B[j][t] for t in range(k)), Fraction(0))
                assert got[r, j] == float(exact)
    with pytest.raises(ValueError):
        O.grouped_gemm_nt(aq, as_, bq, bs, np.array([0, 3, 2, 5, 6]))


# --------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal(200000) * np.ldexp(1.0, rng.integers(-140, 120, 200000))).astype(np.float32)
    # add exact midpoints and tiny subnormals
    x[:1000] = (np.arange(1000, dtype=np.uint32) * 65536 + 0x3F800000 + 0x8000).view(np.float32)
    x[1000:1100] = np.ldexp(np.float32(1.0), -140)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_floored_max_rel():
    r = np.array([1.0, -2.0, 1e-9, 3.0])
    c = r.copy()
    assert O.floored_max_rel(c, r) == 0.0
    c[2] += 1e-3
    rms = math.sqrt(np.mean(r * r))
    assert O.floored_max_rel(c, r) == pytest.approx(1e-3 / rms)
