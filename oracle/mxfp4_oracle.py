"""CPU oracle for the MXFP4 quantize / NT GEMM / grouped NT GEMM path.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, obviously correct
definition that the HIP kernels are checked against.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the C-ABI library and its Python binding) never does, and this
module imports nothing from the product package.

What it follows
---------------
* Formats.  "Packed MXFP4 & NVFP4 GEMM + mega-MoE (SM100, true 2-CTA
  multicast)", Summary: both operands are packed E2M1, two elements per byte,
  and MXFP4 carries UE8M0 scale factors at granularity 32 along K.  The
  "fp4_quantization" Mojo module page (its function list) describes the same
  operand pair for AMD CDNA4: BF16 in, packed MXFP4 with E8M0 block scales out.
  The pages name the formats but print neither the E2M1 value table nor the
  scale rule; the plainest reading is the OCP Microscaling (MX) v1.0
  definition of those formats, restated here from the bit fields:
    - E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no
      Inf/NaN; exponent field 0 is subnormal (value 0.5 * mantissa).
    - E8M0: an unsigned biased exponent, byte b means 2**(b - 127); 255 is NaN.
    - shared exponent of a block: floor(log2(max|x|)) minus the largest
      E2M1 exponent (2), kept inside the E8M0 range.
    - element: x / 2**e rounded to the nearest E2M1 value, ties to the even
      code, magnitudes above 6 saturated to 6.
* Nibble order.  "qgemm-mx" project page, "Where it actually stands": its
  reference kernel reads the packed codes in plain element order; read here
  as element 2j in the low nibble of byte j.
* GEMM.  Same DeepGEMM page, Summary: mxfp4_gemm_nt computes
  [M,K] @ [N,K].T -> [M,N] with BF16 out.  The oracle decodes both operands
  exactly and contracts in float64 (a BLAS matmul on the decoded values).
* Grouped GEMM.  "fp4_quantization" page, grouped_matmul_block_scaled_mxfp4:
  a per-expert grouped MXFP4 matmul; here expert g owns rows
  [offsets[g], offsets[g+1]) of A and its own [N,K] weight.

Pins: every function here is checked in tests/test_oracle_pins.py against
closed forms, exhaustive alternative derivations, brute force with exact
rational arithmetic, and library routines (see that file's docstring).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Element and scale formats
# --------------------------------------------------------------------------

BLOCK = 32          # elements sharing one E8M0 scale (granularity 32 along K)
E2M1_EMAX = 2       # exponent of the largest E2M1 normal (6 = 1.5 * 2**2)
E8M0_BIAS = 127
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code, decoded from its bit fields.

    bit 3 = sign, bits 2..1 = exponent (bias 1), bit 0 = mantissa.
    Exponent field 0 is the subnormal range: 0.5 * mantissa.
    """
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp_field = (code >> 1) & 3
    mant = code & 1
    if exp_field == 0:
        mag = 0.5 * mant
    else:
        mag = 2.0 ** (exp_field - 1) * (1.0 + 0.5 * mant)
    return sign * mag


# decode table built from the bit-field definition above (sign kept on -0)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
# magnitudes of the 8 non-negative codes, in code order
E2M1_MAGNITUDES = E2M1_TABLE[:8].copy()


def e8m0_value(byte) -> np.ndarray:
    """2**(b - 127) for E8M0 bytes; 255 (NaN) is rejected."""
    b = np.asarray(byte, dtype=np.int64)
    if np.any((b < 0) | (b > 254)):
        raise ValueError("E8M0 byte 255 (NaN) or out of range")
    return np.ldexp(1.0, (b - E8M0_BIAS).astype(np.int32))


# --------------------------------------------------------------------------
# BF16 helpers (BF16 is carried as its raw uint16 bit pattern)
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of BF16 bit patterns (upper half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to BF16, nearest-even, returned as uint16 bits.

    Done in exact arithmetic from the float64 value (no intermediate fp32),
    so there is a single rounding.  BF16 has 8 significant bits, exponent
    range as fp32 (normals from 2**-126, subnormal spacing 2**-133).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("non-finite value")
    sign = np.signbit(x)
    a = np.abs(x)
    m, p = np.frexp(a)                      # a = m * 2**p, m in [0.5, 1)
    # quantum: 2**(p - 8) for normals, 2**-133 once p - 8 < -133
    q_exp = np.maximum(p - 8, -133)
    n = np.rint(np.ldexp(a, -q_exp))        # integer multiple of the quantum; rint = ties-to-even
    r = np.ldexp(n, q_exp)
    max_bf16 = float(np.ldexp(255.0, 120))   # (2 - 2**-7) * 2**127
    if np.any(r > max_bf16):
        raise ValueError("overflow to infinity in BF16 rounding")
    r32 = np.where(sign, -r, r).astype(np.float32)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Quantization (BF16 -> packed E2M1 + E8M0), one 32-element block at a time
# --------------------------------------------------------------------------

def shared_exponent(amax) -> np.ndarray:
    """floor(log2(amax)) - 2, clamped to [-127, 127]; amax == 0 gives -127.

    floor(log2) is taken exactly from frexp: amax = m * 2**p with
    m in [0.5, 1), so floor(log2(amax)) = p - 1.
    """
    a = np.asarray(amax, dtype=np.float64)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("amax must be finite and non-negative")
    _, p = np.frexp(a)
    e = (p.astype(np.int64) - 1) - E2M1_EMAX
    e = np.where(a == 0, E8M0_MIN_EXP, e)
    return np.clip(e, E8M0_MIN_EXP, E8M0_MAX_EXP)


def encode_e2m1_magnitude(v) -> np.ndarray:
    """Nearest E2M1 magnitude code (0..7) for v >= 0, by brute-force search.

    Every candidate magnitude is compared; among equally near candidates the
    even code (mantissa bit 0) wins, which is round-to-nearest-even.  Values
    in (6, 8) have 6 as their nearest grid point, which is the saturation.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("magnitude must be finite and non-negative")
    # Inside a block v = |x| / 2**e <= amax / 2**e < 8 (e = floor(log2 amax) - 2,
    # and the lower clamp only makes v smaller).  On [0, 8) the comparison is
    # exact: a v within 0.125 of a grid midpoint has at most 8 significant bits
    # and its lowest bit is at least 2**-10, so both distances are exact in
    # float64; a smaller v is unambiguously nearest to 0.  Far above 8 the
    # distances would round together, hence the domain check.
    if np.any(v >= 8.0):
        raise ValueError("scaled magnitude outside the block range [0, 8)")
    dist = np.abs(v[..., None] - E2M1_MAGNITUDES)          # [..., 8]
    dmin = dist.min(axis=-1, keepdims=True)
    nearest = dist == dmin
    even = nearest & ((np.arange(8) & 1) == 0)
    has_even = even.any(axis=-1)
    pick_even = np.argmax(even, axis=-1)
    pick_any = np.argmax(nearest, axis=-1)
    return np.where(has_even, pick_even, pick_any).astype(np.uint8)


def quantize_block_values(x: np.ndarray):
    """Quantize float64 blocks x[..., 32] (values exactly BF16) -> (codes, scale byte).

    codes: uint8 [..., 32] (4-bit codes, sign in bit 3); scale: uint8 [...].
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != BLOCK:
        raise ValueError("last axis must hold one 32-element block")
    if np.any(~np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the format's definition")
    amax = np.abs(x).max(axis=-1)
    e = shared_exponent(amax)
    v = np.ldexp(np.abs(x), (-e)[..., None].astype(np.int32))   # exact in float64
    mag = encode_e2m1_magnitude(v)
    sign = np.signbit(x).astype(np.uint8) << 3
    codes = (sign | mag).astype(np.uint8)
    scale = (e + E8M0_BIAS).astype(np.uint8)
    return codes, scale


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [..., K] into bytes [..., K/2]; element 2j -> low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("odd number of codes")
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_codes(q: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes: bytes [..., K/2] -> codes [..., K]."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def quantize(x_bits, chunk_rows: int | None = None):
    """BF16 [rows, K] (uint16 bit patterns) -> (q uint8 [rows, K/2], s uint8 [rows, K/32]).

    Rows are processed independently; chunking only bounds memory.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array")
    rows, k = x_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    q = np.empty((rows, k // 2), dtype=np.uint8)
    s = np.empty((rows, k // BLOCK), dtype=np.uint8)
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 20) // max(k, 1))
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        xv = bf16_bits_to_f64(x_bits[r0:r1]).reshape(r1 - r0, k // BLOCK, BLOCK)
        codes, scale = quantize_block_values(xv)
        q[r0:r1] = pack_codes(codes.reshape(r1 - r0, k))
        s[r0:r1] = scale
    return q, s


def dequantize(q, s) -> np.ndarray:
    """(q [rows, K/2], s [rows, K/32]) -> exact float64 values [rows, K]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    rows, half = q.shape
    k = half * 2
    if s.shape != (rows, k // BLOCK):
        raise ValueError("scale shape does not match codes")
    vals = E2M1_TABLE[unpack_codes(q)].reshape(rows, k // BLOCK, BLOCK)
    vals = vals * e8m0_value(s)[..., None]
    return vals.reshape(rows, k)


# --------------------------------------------------------------------------
# GEMMs on the decoded operands
# --------------------------------------------------------------------------

def gemm_nt(a_q, a_s, b_q, b_s) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] * B[n, k] in float64 on exactly decoded operands."""
    a = dequantize(a_q, a_s)
    b = dequantize(b_q, b_s)
    if a.shape[1] != b.shape[1]:
        raise ValueError("K mismatch")
    return a @ b.T


def gemm_nt_f32(a_q, a_s, b_q, b_s) -> np.ndarray:
    """The same contraction accumulated in float32 (summation order left to BLAS).

    The decoded operand values are exact in float32 (|x| between 2**-128 and
    6 * 2**125), so only the accumulation differs from gemm_nt.
    """
    a = dequantize(a_q, a_s).astype(np.float32)
    b = dequantize(b_q, b_s).astype(np.float32)
    return a @ b.T


def grouped_gemm_nt(a_q, a_s, b_q, b_s, offsets) -> np.ndarray:
    """Per-group NT GEMM: rows [offsets[g], offsets[g+1]) of A times B[g].T.

    a_q [total_m, K/2], a_s [total_m, K/32], b_q [G, N, K/2], b_s [G, N, K/32],
    offsets int [G+1] non-decreasing from 0 to total_m.  Returns float64
    [total_m, N]; a group with no rows contributes nothing.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    b_q = np.asarray(b_q, dtype=np.uint8)
    b_s = np.asarray(b_s, dtype=np.uint8)
    groups = b_q.shape[0]
    total_m = np.asarray(a_q).shape[0]
    if offsets.shape != (groups + 1,) or offsets[0] != 0 or offsets[-1] != total_m \
            or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must run from 0 to total_m, non-decreasing, one per group + 1")
    out = np.zeros((total_m, b_q.shape[1]), dtype=np.float64)
    for g in range(groups):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            out[lo:hi] = gemm_nt(np.asarray(a_q)[lo:hi], np.asarray(a_s)[lo:hi], b_q[g], b_s[g])
    return out


def round_output_bf16(c64) -> np.ndarray:
    """The BF16 output format of the GEMM: nearest-even rounding of the exact result."""
    return f64_to_bf16_bits(c64)


# --------------------------------------------------------------------------
# Error metrics used by the parity tests
# --------------------------------------------------------------------------

def floored_max_rel(c, r) -> float:
    """max_i |c_i - r_i| / max(|r_i|, rms(r)).

    Plain elementwise relative error is unbounded for outputs near zero under
    any summation order; flooring the denominator at the RMS of the reference
    keeps the metric meaningful for every element.
    """
    c = np.asarray(c, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if c.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    floor = np.maximum(np.abs(r), rms)
    floor = np.where(floor == 0, 1.0, floor)
    return float(np.max(np.abs(c - r) / floor))
