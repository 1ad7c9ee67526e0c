"""CPU oracle for MXFP8 activations and the W4A8 NT GEMM (MXFP8 A x MXFP4 B).

TEST INFRASTRUCTURE ONLY, like mxfp4_oracle: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it, and it imports
nothing from the product package.

What it follows
---------------
* The "fp4_quantization" Mojo module page lists quantizers that turn BF16 into
  NVFP4, MXFP4 or MXFP8 with per-block scale factors
  (quantize_dynamic_scaled_fp4fp8 and its grouped form) and a block-scaled
  matmul that takes MXFP8 operands (block_scaled_matmul).  The pages name the
  format but print neither its element table nor its scale rule; as for
  MXFP4, the plainest reading is the OCP Microscaling (MX) v1.0 definition,
  restated here from the bit fields:
    - E4M3 element: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
      exponent field 0 is subnormal (mantissa * 2**-9); the code S.1111.111
      is NaN and there is no infinity, so the largest finite magnitude is
      1.75 * 2**8 = 448.
    - shared exponent of a 32-element block: floor(log2(max|x|)) minus the
      largest E4M3 exponent (8), kept inside the E8M0 range (the same E8M0
      scale bytes as MXFP4, one per 32 elements along K).
    - element: x / 2**e rounded to the nearest finite E4M3 value, ties to the
      even code (mantissa bit 0 clear); magnitudes above 448 saturate to 448.
* Storage: one code byte per element, row-major [rows, K]; scales [rows, K/32].
* W4A8 GEMM: C[m, n] = sum_k A[m, k] * B[n, k] with A in MXFP8 and B in
  MXFP4 (packed as in mxfp4_oracle), contracted in float64 on the exactly
  decoded values.
* MXFP8 GEMM: the same contraction with both operands in MXFP8 (the
  block_scaled_matmul entry of the "fp4_quantization" page's Functions list
  takes MXFP8 operands on both sides).

Pins: tests/test_oracle_mxfp8_pins.py checks every function here against
closed forms, PyTorch's float8_e4m3fn conversion (a library routine), exact
rational brute force, an integer matmul and invariants.
"""
from __future__ import annotations

import numpy as np

from .mxfp4_oracle import (BLOCK, E8M0_BIAS, E8M0_MAX_EXP, E8M0_MIN_EXP, bf16_bits_to_f64, dequantize as
                           dequantize_mxfp4, e8m0_value)

E4M3_EMAX = 8           # exponent of the largest E4M3 normal (448 = 1.75 * 2**8)
E4M3_MAX = 448.0
E4M3_NAN_MAG = 0x7F     # S.1111.111


def e4m3_value(code: int) -> float:
    """Value of one 8-bit E4M3 code from its bit fields (NaN for S.1111.111).

    bit 7 = sign, bits 6..3 = exponent (bias 7), bits 2..0 = mantissa.
    """
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("E4M3 code out of range")
    sign = -1.0 if code & 0x80 else 1.0
    mag = code & 0x7F
    if mag == E4M3_NAN_MAG:
        return float("nan")
    e = mag >> 3
    m = mag & 7
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# finite non-negative magnitudes, indexed by magnitude code 0..126
E4M3_MAGNITUDES = E4M3_TABLE[:E4M3_NAN_MAG].copy()


def shared_exponent_e4m3(amax) -> np.ndarray:
    """floor(log2(amax)) - 8, clamped to [-127, 127]; amax == 0 gives -127."""
    a = np.asarray(amax, dtype=np.float64)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("amax must be finite and non-negative")
    _, p = np.frexp(a)                       # a = f * 2**p, f in [0.5, 1)
    e = (p.astype(np.int64) - 1) - E4M3_EMAX
    e = np.where(a == 0, E8M0_MIN_EXP, e)
    return np.clip(e, E8M0_MIN_EXP, E8M0_MAX_EXP)


def encode_e4m3_magnitude(v) -> np.ndarray:
    """Nearest finite E4M3 magnitude code (0..126) for v >= 0, by brute force.

    Every finite magnitude is a candidate; among equally near candidates the
    even code wins (round to nearest even).  Above 448 the nearest finite
    candidate is 448 itself, which is the saturation.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("magnitude must be finite and non-negative")
    # In a block v < 2**9.  A BF16 value scaled by a power of two has at most 8
    # significant bits and the grid at most 4, so on [0, 512) every distance
    # below is exact in float64 and ties are detected exactly.
    if np.any(v >= 512.0):
        raise ValueError("scaled magnitude outside the block range [0, 512)")
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 16
    for i in range(0, flat.size, step):
        part = flat[i:i + step]
        dist = np.abs(part[:, None] - E4M3_MAGNITUDES[None, :])      # [n, 127]
        nearest = dist == dist.min(axis=1, keepdims=True)
        even = nearest & ((np.arange(E4M3_NAN_MAG) & 1) == 0)
        has_even = even.any(axis=1)
        out[i:i + step] = np.where(has_even, np.argmax(even, axis=1), np.argmax(nearest, axis=1))
    return out.reshape(v.shape)


def quantize_block_values_e4m3(x: np.ndarray):
    """Quantize float64 blocks x[..., 32] (values exactly BF16) -> (codes, scale byte)."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != BLOCK:
        raise ValueError("last axis must hold one 32-element block")
    if np.any(~np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the format's definition")
    amax = np.abs(x).max(axis=-1)
    e = shared_exponent_e4m3(amax)
    v = np.ldexp(np.abs(x), (-e)[..., None].astype(np.int32))     # exact in float64
    mag = encode_e4m3_magnitude(v)
    sign = np.signbit(x).astype(np.uint8) << 7
    codes = (sign | mag).astype(np.uint8)
    scale = (e + E8M0_BIAS).astype(np.uint8)
    return codes, scale


def quantize_mxfp8(x_bits, chunk_rows: int | None = None):
    """BF16 [rows, K] (uint16 bit patterns) -> (q uint8 [rows, K], s uint8 [rows, K/32])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array")
    rows, k = x_bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    q = np.empty((rows, k), dtype=np.uint8)
    s = np.empty((rows, k // BLOCK), dtype=np.uint8)
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 18) // max(k, 1))
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        xv = bf16_bits_to_f64(x_bits[r0:r1]).reshape(r1 - r0, k // BLOCK, BLOCK)
        codes, scale = quantize_block_values_e4m3(xv)
        q[r0:r1] = codes.reshape(r1 - r0, k)
        s[r0:r1] = scale
    return q, s


def dequantize_mxfp8(q, s) -> np.ndarray:
    """(q [rows, K], s [rows, K/32]) -> exact float64 values [rows, K]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    rows, k = q.shape
    if s.shape != (rows, k // BLOCK):
        raise ValueError("scale shape does not match codes")
    if np.any((q & 0x7F) == E4M3_NAN_MAG):
        raise ValueError("NaN code in an MXFP8 operand")
    vals = E4M3_TABLE[q].reshape(rows, k // BLOCK, BLOCK) * e8m0_value(s)[..., None]
    return vals.reshape(rows, k)


def gemm_w4a8_nt(a_q8, a_s, b_q, b_s) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] * B[n, k]: A MXFP8 [m, K], B MXFP4 [n, K/2]; float64."""
    a = dequantize_mxfp8(a_q8, a_s)
    b = dequantize_mxfp4(b_q, b_s)
    if a.shape[1] != b.shape[1]:
        raise ValueError("K mismatch")
    return a @ b.T


def gemm_mxfp8_nt(a_q8, a_s, b_q8, b_s) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] * B[n, k]: A MXFP8 [m, K], B MXFP8 [n, K]; float64."""
    a = dequantize_mxfp8(a_q8, a_s)
    b = dequantize_mxfp8(b_q8, b_s)
    if a.shape[1] != b.shape[1]:
        raise ValueError("K mismatch")
    return a @ b.T
