/*
 * mxfp4_producers.h - fused producers of the MI355X (gfx950) MXFP4 library:
 * kernels that compute an activation and write it already quantized to MXFP4
 * (the format of mxfp4.h), so the GEMM that consumes it can run without a
 * separate quantization pass over a BF16 copy.
 *
 * The quadbit README ("Accuracy (real models)", "The stack") runs its FP4
 * transformer block with fused RMSNorm, residual-add and SwiGLU quantizers
 * around the GEMMs.  The pages do not print the operations; the standard
 * definitions are taken, with the BF16 activation the producer would otherwise
 * write as the value that is quantized:
 *   residual add  h = RNE_bf16(x + residual)                 (exact sum, one rounding)
 *   RMSNorm       y = RNE_bf16(h * gamma / sqrt(mean(h^2) + eps))
 *   SwiGLU        y = RNE_bf16(g * u / (1 + exp(-g)))        (silu(g) * u)
 *   then (q, scales) = mxfp4_quantize(y), byte for byte.
 *
 * Conventions of mxfp4.h hold: device pointers on the current device,
 * caller-owned buffers, host-side checks that launch nothing on failure,
 * stream-ordered asynchronous calls with no allocation, mxfp4_last_error()
 * for details, gfx950 only.  BF16 arrays are 16-byte aligned; q 4-byte
 * aligned; scales any alignment.
 */
#ifndef MXFP4_PRODUCERS_H_
#define MXFP4_PRODUCERS_H_

#include <stddef.h>
#include <stdint.h>

#include "mxfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Residual add + RMSNorm + MXFP4 quantization, one row at a time.
 *   x_bf16 [rows, k]; residual_bf16 [rows, k] or NULL (then h = x);
 *   gamma_bf16 [k]; eps >= 0 (finite);
 *   residual_out_bf16 [rows, k] or NULL: receives h (the updated residual
 *     stream; only written when residual_bf16 is given; may be the same buffer
 *     as residual_bf16 or x_bf16);
 *   y_bf16 [rows, k] or NULL: receives the BF16 RMSNorm output (may be the
 *     same buffer as x_bf16);
 *   q [rows, k/2], scales [rows, k/32]: MXFP4 of y.
 * Arithmetic: h in fp32 then nearest-even BF16 (equal to rounding the exact
 * sum); the sum of squares and y = (h * inv) * gamma with
 * inv = 1 / sqrt(sum / k + eps) in fp64, y rounded once to BF16.  y therefore
 * equals the nearest BF16 of the exact value except where that value lies
 * within about 2^-50 (relative) of a BF16 rounding midpoint.
 * Limits: k a positive multiple of 32, k <= 32768; 0 <= rows <= 2^24 (one
 * workgroup per row); rows == 0 is a no-op.
 */
mxfp4_status_t mxfp4_rmsnorm_quantize(const void* x_bf16, const void* residual_bf16, const void* gamma_bf16,
                                      float eps, int64_t rows, int64_t k, void* residual_out_bf16, void* y_bf16,
                                      void* q, void* scales, void* stream);

/*
 * SwiGLU + MXFP4 quantization: y[r, i] = silu(gate[r, i]) * up[r, i] for
 * i < k, read with row stride ld (elements) from both inputs, so a fused
 * [rows, 2k] gate|up projection passes gate = base, up = base + k, ld = 2k.
 *   gate_bf16, up_bf16: rows of ld elements (16-byte aligned, ld % 8 == 0,
 *     ld >= k);
 *   y_bf16 [rows, k] or NULL: receives the BF16 activation;
 *   q [rows, k/2], scales [rows, k/32]: MXFP4 of y.
 * Arithmetic: (g * u) * rcp(1 + exp2(-g * log2 e)) in fp32 with the hardware
 * exp2 and reciprocal (relative error at most about (|g| + 6) * 2^-24), then
 * nearest-even BF16; y is within one BF16 step of the exact value and equals
 * its nearest BF16 except that close to a rounding midpoint.
 * Limits: k a positive multiple of 32, rows * k / 32 <= 2^30; rows == 0 is a
 * no-op.
 */
mxfp4_status_t mxfp4_swiglu_quantize(const void* gate_bf16, const void* up_bf16, int64_t ld, int64_t rows,
                                     int64_t k, void* y_bf16, void* q, void* scales, void* stream);

/*
 * The two producers with their MXFP4 output stored in the prepacked operand
 * layout of mxfp4_gemm_nt_prepacked_ab (include/mxfp4.h, the layout of
 * mxfp4_prepack_weight applied to [rows, k]): the quantization fused into the
 * activation's producer, so the small-M (decode) GEMM on prepacked operands
 * follows the producer with no quantization launch in between (the quadbit
 * README, "The stack": producers that quantize in place; the "Packed MXFP4 &
 * NVFP4 GEMM + mega-MoE" page, Summary: the decode GEMM's activation
 * operand).  The code and scale bytes are those of mxfp4_rmsnorm_quantize /
 * mxfp4_swiglu_quantize, byte for byte, at the positions the layout gives
 * them; rows from `rows` up to the next multiple of 64 are written as zero
 * blocks (code 0, scale byte 0), as mxfp4_quantize_prepacked writes them.
 *   ap_q, ap_s : device buffers of the sizes mxfp4_prepacked_weight_size(rows,
 *                k) gives (ap_q 16-byte aligned);
 *   k          : a positive multiple of 512 (MXFP4_ERR_INVALID_ARG otherwise).
 * Every other argument, limit and result as for the row-major producers above.
 */
mxfp4_status_t mxfp4_rmsnorm_quantize_prepacked(const void* x_bf16, const void* residual_bf16,
                                                const void* gamma_bf16, float eps, int64_t rows, int64_t k,
                                                void* residual_out_bf16, void* y_bf16, void* ap_q, void* ap_s,
                                                void* stream);

mxfp4_status_t mxfp4_swiglu_quantize_prepacked(const void* gate_bf16, const void* up_bf16, int64_t ld, int64_t rows,
                                               int64_t k, void* y_bf16, void* ap_q, void* ap_s, void* stream);

/*
 * The two producers with their scale bytes in the interleaved layout of
 * include/mxfp4.h (scales_il [k/512, rows, 16]), the A operand scales of
 * mxfp4_gemm_nt_interleaved: a prefill activation produced and quantized in
 * one launch for the tile GEMM's faster scale layout (the "fp4_quantization"
 * page, grouped_quantize_dynamic_scaled_fp4_async: scales written in the
 * matrix path's order as they are produced).  Codes q [rows, k/2] row-major;
 * codes, scale values and the BF16 outputs those of mxfp4_rmsnorm_quantize /
 * mxfp4_swiglu_quantize, byte for byte.  k a positive multiple of 512 and
 * rows * k / 32 < 2^31 (MXFP4_ERR_INVALID_ARG otherwise); every other
 * argument, limit and result as for the row-major producers.
 */
mxfp4_status_t mxfp4_rmsnorm_quantize_interleaved(const void* x_bf16, const void* residual_bf16,
                                                  const void* gamma_bf16, float eps, int64_t rows, int64_t k,
                                                  void* residual_out_bf16, void* y_bf16, void* q, void* scales_il,
                                                  void* stream);

mxfp4_status_t mxfp4_swiglu_quantize_interleaved(const void* gate_bf16, const void* up_bf16, int64_t ld,
                                                 int64_t rows, int64_t k, void* y_bf16, void* q, void* scales_il,
                                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_PRODUCERS_H_ */
