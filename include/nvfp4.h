/*
 * nvfp4.h - NVFP4 operands of the MI355X (gfx950) library: packed E2M1 codes
 * with UE4M3 scales per 16 elements and an fp32 global scale per row, their
 * dynamic quantization from BF16, and the NT GEMM on two NVFP4 operands.
 *
 * The "Packed MXFP4 & NVFP4 GEMM + mega-MoE" page (Summary) defines NVFP4 as
 * packed E2M1 with E4M3/UE4M3 scale factors at granularity 16 plus global
 * scales, the GEMM result being acc * gs_act * gs_weight (nvfp4_gemm_nt:
 * [M,K] @ [N,K].T -> [M,N], BF16 out); the quadbit README ("Accuracy (real
 * models)") uses the two-level form with a per-row fp32 global scale, which is
 * the form here (a per-tensor scale is the case of equal entries).
 *
 * Layout of an NVFP4 operand of rows x k elements (row-major, K innermost):
 *   q      uint8 [rows, k/2]   E2M1 codes, element 2j in the low nibble of byte j;
 *   scales uint8 [rows, k/16]  UE4M3 codes (bits 6..3 exponent, bias 7; bits 2..0
 *                              mantissa; exponent 0 is subnormal, m * 2^-9;
 *                              never 0x7F or above);
 *   gs     float [rows]        global scale of each row.
 * Element value: e2m1(code) * ue4m3(scale of its 16-block) * gs[row].
 *
 * Conventions of mxfp4.h hold (device pointers, caller-owned buffers,
 * host-side checks that launch nothing on failure, stream-ordered
 * asynchronous calls with no allocation, mxfp4_last_error(), gfx950 only).
 *
 * gfx950 note: the scaled f8f6f4 MFMA takes E8M0 scales that each cover 32
 * elements and cannot apply 16-element UE4M3 scales, so the NVFP4 GEMM
 * dequantizes each stage exactly to BF16 in LDS (e2m1 * ue4m3 has at most 6
 * significant bits) and runs on the BF16 MFMA: a quarter of the FP4 MFMA rate.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#include "mxfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Dynamic BF16 -> NVFP4 quantization, one row at a time.  Every step is an
 * IEEE fp32 operation:
 *   A  = max |x| of the row;  gs = A / 2688 (6 * 448), or 1 when A == 0;
 *   per 16-element block: t = amax / (6 * gs); s = t rounded to the nearest
 *   UE4M3 value (ties to the even code, saturated at 448); d = s * gs;
 *   code = sign(x) | (|x| / d rounded to the nearest E2M1 magnitude, ties to
 *   the even code, saturated at 6); a block with d == 0 (s == 0, or s * gs
 *   underflowing) encodes signed zeros.
 * x_bf16 [rows, k] (16-byte aligned); q [rows, k/2] (4-byte aligned); scales
 * [rows, k/16] (any alignment); global_scales [rows] (4-byte aligned).
 * Limits: k a positive multiple of 32, k <= 32768; 0 <= rows <= 2^24 (one
 * workgroup per row); rows == 0 is a no-op.
 */
mxfp4_status_t nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t k, void* q, void* scales,
                              float* global_scales, void* stream);

/*
 * NVFP4 NT GEMM: C[m][n] = (acc[m][n] * a_gs[m]) * b_gs[n] with
 * acc = sum_k e2m1(a) ue4m3(a's block) e2m1(b) ue4m3(b's block), products
 * exact (BF16 MFMA on exactly dequantized operands) and accumulated in fp32;
 * C is BF16 (nearest-even) or fp32 by c_type.
 *   a_q [m, k/2], a_s [m, k/16], a_gs [m];  b_q [n, k/2], b_s [n, k/16], b_gs [n];
 *   code arrays 16-byte aligned, scale arrays and global scales 4-byte aligned,
 *   c [m, n] 16-byte aligned.
 * Limits: k a positive multiple of 64, k <= 2^24; m, n <= 2^30; m == 0 or
 * n == 0 is a no-op.
 */
mxfp4_status_t nvfp4_gemm_nt(const void* a_q, const void* a_s, const float* a_gs, const void* b_q, const void* b_s,
                             const float* b_gs, void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
