/*
 * mxfp8.h - MXFP8 activations of the MI355X (gfx950) MXFP4 library: the
 * activation format of a W4A8 GEMM, MXFP8 (E4M3) activations times MXFP4
 * (E2M1) weights.
 *
 * The "fp4_quantization" Mojo module page lists quantizers that turn BF16
 * into NVFP4, MXFP4 or MXFP8 with per-block scale factors
 * (quantize_dynamic_scaled_fp4fp8) and a block-scaled matmul that takes MXFP8
 * operands (block_scaled_matmul).  The format follows the OCP MX definition:
 *   - q8     uint8 [rows, k]     one E4M3 code per element: bit 7 sign,
 *                                bits 6..3 exponent (bias 7), bits 2..0
 *                                mantissa; largest finite magnitude 448;
 *                                S.1111.111 (NaN) is never produced;
 *   - scales uint8 [rows, k/32]  one E8M0 byte per 32 consecutive elements
 *                                (byte b means 2^(b-127)), as for MXFP4.
 * Weights stay MXFP4 exactly as in mxfp4.h.  The conventions of mxfp4.h hold
 * (device pointers on the current device, caller-owned buffers, host-side
 * checks that launch nothing on failure, stream-ordered asynchronous calls,
 * mxfp4_last_error() for details, gfx950 only).
 */
#ifndef MXFP8_H_
#define MXFP8_H_

#include <stddef.h>
#include <stdint.h>

#include "mxfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Dynamic block-scaled quantization BF16 -> MXFP8.  For each row and each
 * 32-element block along K:
 *   amax = max |x_i|;
 *   e = floor(log2 amax) - 8 (8 is the exponent of E4M3's largest value 448),
 *       clamped to [-127, 127]; an all-zero block gets e = -127;
 *   scale byte = e + 127;
 *   code_i = x_i / 2^e rounded to the nearest E4M3 value, ties to the even
 *            code, magnitudes above 448 saturated to 448; a negative input
 *            keeps its sign bit (-0 encodes as 0x80).
 * x_bf16 [rows, k] row-major, 16-byte aligned; q8 [rows, k], 8-byte aligned;
 * scales [rows, k/32], any alignment.  k a positive multiple of 32,
 * k <= 2^24, rows * k <= 2^40; rows == 0 is a no-op.
 */
mxfp4_status_t mxfp8_quantize(const void* x_bf16, int64_t rows, int64_t k, void* q8, void* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H_ */
