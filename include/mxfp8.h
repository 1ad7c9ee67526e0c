/*
 * mxfp8.h - MXFP8 activations and W4A8 GEMMs of the MI355X (gfx950) MXFP4
 * library: MXFP8 (E4M3) activations times MXFP4 (E2M1) weights.
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

/*
 * W4A8 NT GEMM: C[m][n] = sum_k A[m][k] * B[n][k] with A in MXFP8 and B in
 * MXFP4 ("fp4_quantization" page, block_scaled_matmul: block-scaled matmul
 * over MXFP4 / MXFP8 operands), on the scaled MFMA with fp32 accumulation; C
 * is written as BF16 (nearest-even) or fp32 by c_type, as in mxfp4_gemm_nt.
 * Numerics: with an FP8 operand the gfx950 MFMA sums each aligned group of 8
 * products along K after aligning them to the group's largest exponent sum E
 * (E4M3 plus E2M1 exponent) and truncating each toward zero to a multiple of
 * 2^(E-13) (measured; FP4 x FP4 products always lie on that grid).  So C
 * differs from the exact sum by less than, per group, (nonzero products) x
 * 2^(E-13) x the two block scales, plus fp32 accumulation rounding.
 *   a_q8 [m, k]    E4M3 codes;   a_s [m, k/32] E8M0 bytes;
 *   b_q  [n, k/2]  packed E2M1;  b_s [n, k/32] E8M0 bytes (layout of mxfp4.h);
 *   c    [m, n].
 * k a positive multiple of 32, k <= 2^24; m, n <= 2^30; m == 0 or n == 0 is a
 * no-op.  Alignment as in mxfp4.h (codes and c 16 bytes; scale arrays 4 bytes
 * when k % 128 == 0).  The fast paths take k % 512 == 0 with 16-byte aligned
 * scale arrays.  Codes S.1111.111 (NaN) in A are outside the format: the
 * result is then unspecified.  No workspace; one kernel launch.
 */
mxfp4_status_t mxfp8_gemm_w4a8_nt(const void* a_q8, const void* a_s, const void* b_q, const void* b_s, void* c,
                                  mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * mxfp8_gemm_w4a8_nt with the kernel forced, for tests and tuning:
 *   MXFP4_KERNEL_AUTO     the choice mxfp8_gemm_w4a8_nt makes: the streaming
 *                         kernel for m <= 128 when k % 512 == 0 and both scale
 *                         arrays are 16-byte aligned, else the tile kernel;
 *   MXFP4_KERNEL_TILE128  128 x 256 output tiles, LDS-staged scaled MFMA;
 *   MXFP4_KERNEL_STREAM   weight-streaming kernel (32- or 64-row M tiles, 64
 *                         columns, whole K); needs k % 512 == 0 and 16-byte
 *                         aligned scale arrays, any m.
 * Other kernel ids are rejected (MXFP4_ERR_INVALID_ARG).
 */
mxfp4_status_t mxfp8_gemm_w4a8_nt_ex(const void* a_q8, const void* a_s, const void* b_q, const void* b_s, void* c,
                                     mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel,
                                     void* stream);

/*
 * mxfp8_gemm_w4a8_nt on a prepacked weight: bp_q / bp_s are B rearranged by
 * mxfp4_prepack_weight (include/mxfp4.h), so each wave loads B straight into
 * registers; A (MXFP8) goes through LDS as in the streaming kernel, in
 * 128-row tiles for m up to 128 (one workgroup per 64 columns: a single
 * round of workgroups at the decode shape).  The same numerics and, output
 * for output, the same result bit for bit as mxfp8_gemm_w4a8_nt_ex with
 * MXFP4_KERNEL_STREAM (same per-wave K split, MFMA order and reduction).
 * a_q8, a_s: A as in mxfp8_gemm_w4a8_nt, 16-byte aligned; c: [m, n] of type
 * c_type, 16-byte aligned; k a positive multiple of 512, at most 2^24
 * (MXFP4_ERR_INVALID_ARG otherwise).  No workspace; one kernel launch.
 */
mxfp4_status_t mxfp8_gemm_w4a8_nt_prepacked(const void* a_q8, const void* a_s, const void* bp_q, const void* bp_s,
                                            void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                                            void* stream);

/*
 * Both W4A8 operands prepacked: the decode GEMM with the activation also in a
 * prepacked layout, so every wave loads A straight into registers as well and
 * the main loop touches no LDS (the FP8 counterpart of
 * mxfp4_gemm_nt_prepacked_ab; the quadbit README's "The stack": the
 * activation quantized straight into the layout the GEMM reads).
 *
 * FP8 prepacked layout of an MXFP8 operand [rows, k] (k % 512 == 0), per
 * 64-row panel P and 512-K pair t (rows padded to a multiple of 64 with zero
 * blocks): the scaled MFMA's FP8 operand takes, in lane half h of a 64-K step,
 * the codes at K [16h, 16h + 16) in its first four registers and at
 * [32 + 16h, 48 + 16h) in its last four.  For wave w (64-K step w of each
 * 256-K stage s), u = 2s + j (32-row block j of the panel), register half e
 * and lane l = r % 32 + 32h, the 16 codes sit at byte
 *   (P * pairs + t) * 32768 + w * 8192 + u * 2048 + e * 1024 + l * 16
 * of ap_q8: codes of row 64P + 32j + l % 32 at K 512t + 256s + 64w + 32e +
 * 16h + [0, 16).  The scale bytes sit exactly where mxfp4_prepack_weight's
 * layout keeps an MXFP4 operand's (include/mxfp4.h).  Sizes: ap_q8 twice the
 * code bytes mxfp4_prepacked_weight_size(rows, k) gives, ap_s the same scale
 * bytes.
 *
 * mxfp8_quantize_prepacked: mxfp8_quantize with the codes and scale bytes
 *   stored in that layout, bit for bit the same bytes (padding rows zero);
 *   ap_q8 16-byte aligned; k a positive multiple of 512, at most 2^24.
 * mxfp8_gemm_w4a8_nt_prepacked_ab: C[m, n] = A . B^T with A in the FP8
 *   prepacked layout (m rows) and B prepacked by mxfp4_prepack_weight (n rows);
 *   the same result, bit for bit, as mxfp8_gemm_w4a8_nt_prepacked on the
 *   row-major A (same per-wave K split, MFMA order and reduction).  c: [m, n]
 *   of type c_type, 16-byte aligned; k as above.  No workspace; one launch.
 * Violations return MXFP4_ERR_INVALID_ARG.
 */
mxfp4_status_t mxfp8_quantize_prepacked(const void* x_bf16, int64_t rows, int64_t k, void* ap_q8, void* ap_s,
                                        void* stream);

mxfp4_status_t mxfp8_gemm_w4a8_nt_prepacked_ab(const void* ap_q8, const void* ap_s, const void* bp_q,
                                               const void* bp_s, void* c, mxfp4_out_t c_type, int64_t m, int64_t n,
                                               int64_t k, void* stream);

/*
 * MXFP8 x MXFP8 NT GEMM: C[m][n] = sum_k A[m][k] * B[n][k] with both operands
 * in MXFP8 ("fp4_quantization" page, Functions: block_scaled_matmul, the
 * block-scaled matmul over MXFP4 / MXFP8 operands; its quantizer
 * quantize_dynamic_scaled_fp4fp8 produces MXFP8), on the scaled MFMA with
 * both operand formats set to FP8 E4M3 and fp32 accumulation; C is written as
 * BF16 (nearest-even) or fp32 by c_type, as in mxfp4_gemm_nt.
 * Numerics (measured on gfx950): the MFMA sums each aligned group of 8
 * products along K after aligning them to the group's largest exponent sum E
 * (A's plus B's E4M3 exponent) and truncating each toward zero to a multiple
 * of 2^(E-13); within one 64-deep MFMA the group sums are aligned to the
 * largest exponent sum E' of its products and rounded down to a multiple of
 * 2^(E'-24); that sum meets the fp32 accumulator with one nearest-even
 * rounding.  So C differs from the exact sum by less than, per group,
 * (nonzero products) x 2^(E-13), plus per 64-deep step 8 x 2^(E'-24), each
 * times the block scales, plus fp32 accumulation rounding.
 *   a_q8 [m, k]  E4M3 codes;  a_s [m, k/32] E8M0 bytes;
 *   b_q8 [n, k]  E4M3 codes;  b_s [n, k/32] E8M0 bytes;
 *   c    [m, n].
 * k a positive multiple of 32, k <= 2^23 (a 256-row tile of FP8 codes stays
 * below 2^31 bytes); m, n <= 2^30; m == 0 or n == 0 is a no-op.  Alignment as
 * in mxfp4.h (codes and c 16 bytes; scale arrays 4 bytes when k % 128 == 0).
 * The 256 x 256 kernel takes k % 512 == 0 with 16-byte aligned scale arrays;
 * other k run 128 x 128 tiles.  Codes S.1111.111 (NaN) are outside the format:
 * the result is then unspecified.  No workspace; one kernel launch.
 */
mxfp4_status_t mxfp8_gemm_nt(const void* a_q8, const void* a_s, const void* b_q8, const void* b_s, void* c,
                             mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * mxfp8_gemm_nt with the tile size forced, for tests and tuning:
 *   MXFP4_KERNEL_AUTO     the choice mxfp8_gemm_nt makes: 256 x 256 tiles when
 *                         there are at least as many of them as compute units,
 *                         else 128 x 128;
 *   MXFP4_KERNEL_TILE256  256 x 256 output tiles (4 waves of 128 x 128), when
 *                         k % 512 == 0 and the scale arrays are 16-byte
 *                         aligned; otherwise 128 x 128;
 *   MXFP4_KERNEL_TILE128  128 x 128 output tiles.
 * Other kernel ids are rejected (MXFP4_ERR_INVALID_ARG).
 */
mxfp4_status_t mxfp8_gemm_nt_ex(const void* a_q8, const void* a_s, const void* b_q8, const void* b_s, void* c,
                                mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel,
                                void* stream);

/*
 * Grouped per-expert W4A8 NT GEMM: as mxfp4_grouped_gemm_nt with A in MXFP8
 * ([total_m, k] codes, [total_m, k/32] scales), B in MXFP4 ([num_groups, n,
 * k/2], [num_groups, n, k/32]) and the same device `offsets` contract
 * (offsets clamped into [0, total_m] and replaced by their running maximum,
 * so groups are disjoint and in range; a group with no rows writes nothing);
 * num_groups 1..1024.  No workspace; one kernel launch of 128 x 256 tiles,
 * through the persistent tile loop when k % 1024 == 0 and the scale arrays
 * are 16-byte aligned.  Each group's rows equal mxfp8_gemm_w4a8_nt_ex with
 * MXFP4_KERNEL_TILE128 on that group's slices, bit for bit.
 */
mxfp4_status_t mxfp8_grouped_gemm_w4a8_nt(const void* a_q8, const void* a_s, const void* b_q, const void* b_s,
                                          const int32_t* offsets, int32_t num_groups, int64_t total_m, void* c,
                                          mxfp4_out_t c_type, int64_t n, int64_t k, void* stream);

/*
 * The MXFP8 and W4A8 tile GEMMs on interleaved scales: the interleaved layout
 * of include/mxfp4.h ([k/512, rows, 16] per operand: the sixteen scale bytes
 * of a 512-wide K slab of a row next to the next row's; mxfp4_scales_interleave
 * converts row-major scales, and the quantizers below write it directly) for
 * the MXFP8 operands as for the MXFP4 ones.  Same values, bit-identical results
 * to the row-major entry points on the same tile kernels.
 *
 * mxfp8_quantize_interleaved: mxfp8_quantize with the scales written
 *   interleaved (codes as mxfp8_quantize).
 * mxfp8_gemm_w4a8_nt_interleaved: mxfp8_gemm_w4a8_nt_ex with
 *   MXFP4_KERNEL_TILE128 (128 x 256 tiles) at every m, both scale arrays
 *   interleaved.
 * mxfp8_grouped_gemm_w4a8_nt_interleaved: mxfp8_grouped_gemm_w4a8_nt with
 *   a_s_il over total_m rows and b_s_il interleaved per group.
 * mxfp8_gemm_nt_interleaved: mxfp8_gemm_nt (MXFP8 x MXFP8) with both scale
 *   arrays interleaved; the same tile choice.
 * Limits: k a positive multiple of 512 (MXFP8 x MXFP8: at most 2^23, else
 * 2^24); m * k / 32 and n * k / 32 (total_m * k / 32) below 2^31; scale arrays
 * 16-byte aligned; every other argument as for the row-major entry point.
 * Violations return MXFP4_ERR_INVALID_ARG.
 */
mxfp4_status_t mxfp8_quantize_interleaved(const void* x_bf16, int64_t rows, int64_t k, void* q8, void* scales_il,
                                          void* stream);

mxfp4_status_t mxfp8_gemm_w4a8_nt_interleaved(const void* a_q8, const void* a_s_il, const void* b_q,
                                              const void* b_s_il, void* c, mxfp4_out_t c_type, int64_t m, int64_t n,
                                              int64_t k, void* stream);

mxfp4_status_t mxfp8_grouped_gemm_w4a8_nt_interleaved(const void* a_q8, const void* a_s_il, const void* b_q,
                                                      const void* b_s_il, const int32_t* offsets, int32_t num_groups,
                                                      int64_t total_m, void* c, mxfp4_out_t c_type, int64_t n,
                                                      int64_t k, void* stream);

mxfp4_status_t mxfp8_gemm_nt_interleaved(const void* a_q8, const void* a_s_il, const void* b_q8, const void* b_s_il,
                                         void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H_ */
