"""CPU oracle for NVFP4: E2M1 elements, UE4M3 scales per 16 elements and an fp32
global scale per row, and the NT GEMM on two such operands.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library and imports nothing from the product package.

What it follows
---------------
* Format.  "Packed MXFP4 & NVFP4 GEMM + mega-MoE" page, Summary: NVFP4 operands
  are packed E2M1 (two elements per byte) with E4M3/UE4M3 scale factors at
  granularity 16 plus a global scale, and the GEMM result is dequantized as
  acc * gs_act * gs_weight.  The quadbit README ("Accuracy (real models)")
  describes the two-level recipe as a per-16 UE4M3 local scale with a per-row
  fp32 global scale; that per-row form is taken here (a per-tensor global
  scale is the special case of equal rows).
* The pages print no quantization rule.  The plainest reading, each step an
  IEEE fp32 operation so that it is reproducible bit for bit:
    A     = max |x| over the row (exact);
    gs    = fp32(A / 2688), or 1 when A == 0   (2688 = 6 * 448: the largest
            E2M1 magnitude times the largest E4M3 value, so the largest block
            scale lands on 448);
    per 16-element block:
    t     = fp32(amax_block / fp32(6 * gs));
    s     = t rounded to the nearest UE4M3 value (ties to the even code),
            saturated at 448; the block's scale byte is its code;
    d     = fp32(s * gs);
    code  = sign(x) | E2M1 magnitude code of fp32(|x| / d), nearest with ties
            to the even code, saturated at 6; a block whose scale is 0 (or whose
            d underflows to 0) encodes every element as a (signed) zero.
  Dequantization: x = e2m1(code) * s * gs, exact in float64.
* GEMM: C[m, n] = sum_k A[m, k] * B[n, k] on the dequantized operands, float64.
"""
from __future__ import annotations

import numpy as np

from .mxfp4_oracle import E2M1_TABLE, bf16_bits_to_f64, encode_e2m1_magnitude, pack_codes, unpack_codes
from .mxfp8_oracle import E4M3_TABLE, encode_e4m3_magnitude

NVFP4_BLOCK = 16
GLOBAL_DIVISOR = np.float32(6.0 * 448.0)


def global_scales(x_bits) -> np.ndarray:
    """Per-row fp32 global scale gs = fp32(amax / 2688), 1 for an all-zero row."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)        # BF16 values are exact in float32
    amax = np.max(np.abs(x), axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        gs = (amax / GLOBAL_DIVISOR).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), gs).astype(np.float32)


def quantize_nvfp4(x_bits):
    """BF16 [rows, K] (uint16 bits) -> (q uint8 [rows, K/2], s uint8 [rows, K/16], gs float32 [rows])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, k = x_bits.shape
    if k % NVFP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    x = bf16_bits_to_f64(x_bits).astype(np.float32)
    if np.any(~np.isfinite(x)):
        raise ValueError("NaN/Inf input is outside the format's definition")
    gs = global_scales(x_bits)
    blocks = x.reshape(rows, k // NVFP4_BLOCK, NVFP4_BLOCK)
    amax_b = np.max(np.abs(blocks), axis=2)                                   # float32, exact
    six_gs = (np.float32(6.0) * gs).astype(np.float32)                         # fp32(6 * gs)
    t = (amax_b / six_gs[:, None]).astype(np.float32)                          # fp32 quotient
    # t <= 448 * (1 + a few ulps): inside encode_e4m3_magnitude's exact domain [0, 512)
    s_code = encode_e4m3_magnitude(t.astype(np.float64)).astype(np.uint8)
    s_val = E4M3_TABLE[s_code].astype(np.float32)                              # exact
    d = (s_val * gs[:, None]).astype(np.float32)                               # fp32(s * gs)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (np.abs(blocks) / d[:, :, None]).astype(np.float32)                # fp32(|x| / d)
    # a zero scale, or a scale whose product with gs underflows to zero, encodes signed zeros
    v = np.where((s_val[:, :, None] == 0) | (d[:, :, None] == 0), np.float32(0.0), v)
    v = np.minimum(v, np.float32(6.0))                                         # saturation at 6
    mag = encode_e2m1_magnitude(v.astype(np.float64))
    sign = (np.signbit(blocks).astype(np.uint8) << 3)
    codes = (sign | mag).reshape(rows, k).astype(np.uint8)
    return pack_codes(codes), s_code.reshape(rows, k // NVFP4_BLOCK), gs


def dequantize_nvfp4(q, s, gs) -> np.ndarray:
    """(q [rows, K/2], s [rows, K/16] UE4M3 codes, gs [rows] fp32) -> exact float64 [rows, K]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    rows, half = q.shape
    k = half * 2
    if s.shape != (rows, k // NVFP4_BLOCK) or np.any(s >= 0x7F):
        raise ValueError("scale shape or code (UE4M3: 0..126) invalid")
    vals = E2M1_TABLE[unpack_codes(q)].reshape(rows, k // NVFP4_BLOCK, NVFP4_BLOCK)
    vals = vals * E4M3_TABLE[s][..., None] * np.asarray(gs, dtype=np.float64)[:, None, None]
    return vals.reshape(rows, k)


def gemm_nvfp4_nt(a_q, a_s, a_gs, b_q, b_s, b_gs) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] * B[n, k] on exactly dequantized NVFP4 operands, float64."""
    a = dequantize_nvfp4(a_q, a_s, a_gs)
    b = dequantize_nvfp4(b_q, b_s, b_gs)
    if a.shape[1] != b.shape[1]:
        raise ValueError("K mismatch")
    return a @ b.T
