/*
 * mxfp4_moe.h - MoE steps around the grouped MXFP4 GEMM of the MI355X
 * (gfx950) library: top-k routing, the expert-sorted row permutation,
 * quantization scattered into the grouped GEMM's operand rows, and the
 * weighted combine of the expert outputs.
 *
 * What the pages give and the readings taken:
 *   - the grouped GEMM owns one contiguous segment of rows per expert, in a
 *     single launch (quadbit README, "Distributed sparse-FP4 MoE": a segmented
 *     routed-row kernel), and its activation operand is the per-expert
 *     dynamically quantized tile ("fp4_quantization" Mojo module page,
 *     grouped_quantize_dynamic_scaled_fp4_async); the DeepGEMM page (Summary,
 *     mega-MoE) fuses dispatch, the expert GEMMs and combine;
 *   - the pages print no router (the quadbit README keeps it dense and outside
 *     the FP4 path).  Taken here: a token's experts are its k largest logits,
 *     equal logits going to the lower expert id; gate weights are the softmax
 *     of the k selected logits (they sum to 1);
 *   - rows are ordered by (expert, token, slot): the rows of one expert are in
 *     ascending token order, so every result is independent of timing;
 *   - an expert id outside [0, experts) drops its entry: it gets no row and
 *     contributes nothing to the combine.
 *
 * Layouts (row-major, device memory, caller-owned):
 *   logits      float [tokens, experts]
 *   topk_ids    int32 [tokens, top_k]    expert of slot j of token t
 *   topk_weights float [tokens, top_k]   gate weight of that slot
 *   offsets     int32 [experts + 1]      rows of expert e: [offsets[e], offsets[e+1])
 *   row_token   int32 [tokens * top_k]   token of each row; -1 past offsets[experts]
 *   token_rows  int32 [tokens, top_k]    row of each slot; -1 for a dropped slot
 * offsets, the activation operand's rows and the grouped GEMM's output rows
 * are exactly what mxfp4_grouped_gemm_nt (mxfp4.h) takes.
 *
 * Conventions of mxfp4.h hold: host-side argument checks that launch nothing
 * on failure, stream-ordered asynchronous calls with no allocation,
 * mxfp4_last_error() for details, gfx950 only.  Index arrays and float arrays
 * need 4-byte alignment unless stated.  Device-resident indices cannot be
 * checked on the host: every kernel skips a row index outside [0, total_rows),
 * so malformed indices never write outside the given buffers (the result is
 * then unspecified).
 */
#ifndef MXFP4_MOE_H_
#define MXFP4_MOE_H_

#include <stddef.h>
#include <stdint.h>

#include "mxfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Top-k routing.  For each token: the k largest of its `experts` logits in
 * descending order (equal logits: lower expert id first; -0 and +0 are equal)
 * go to topk_ids[t, 0..k-1], and topk_weights[t, j] = exp(l_j - l_0) /
 * sum_i exp(l_i - l_0) over the selected logits, in fp32.  NaN logits give
 * unspecified (but valid and distinct) ids.
 * Limits: 1 <= experts <= 256, 1 <= top_k <= min(8, experts),
 * 0 <= tokens <= 2^28; tokens == 0 is a no-op.
 */
mxfp4_status_t mxfp4_moe_route(const float* logits, int64_t tokens, int32_t experts, int32_t top_k,
                               int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * Expert-sorted permutation of the routed entries (a counting sort, stable in
 * (token, slot) order).  Writes offsets [experts + 1], row_token
 * [tokens * top_k] and token_rows [tokens, top_k] as laid out above; kept
 * entries fill rows [0, offsets[experts]).
 * Limits: 1 <= experts <= 1024, 1 <= top_k <= 256, tokens >= 0,
 * tokens * top_k <= 2^30.  tokens == 0 still writes offsets (all zero).
 */
mxfp4_status_t mxfp4_moe_permute(const int32_t* topk_ids, int64_t tokens, int32_t experts, int32_t top_k,
                                 int32_t* offsets, int32_t* row_token, int32_t* token_rows, void* stream);

/*
 * Dynamic MXFP4 quantization of the token rows, scattered to the routed rows:
 * for every slot (t, j) with r = token_rows[t, j] in [0, total_rows), row r of
 * (q, scales) becomes the MXFP4 quantization of x row t, exactly as
 * mxfp4_quantize would produce it.  Each token row is read and quantized
 * once.  Rows no slot points at are left untouched.
 *   x_bf16 [tokens, k] (16-byte aligned); q [total_rows, k/2] (4-byte
 *   aligned); scales [total_rows, k/32] (any alignment).
 * Limits: k a positive multiple of 32, k <= 2^24; tokens * k / 32 <= 2^30;
 * 1 <= top_k <= 256; 0 <= total_rows < 2^31.  tokens == 0 or
 * total_rows == 0 is a no-op.
 */
mxfp4_status_t mxfp4_moe_quantize_scatter(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                          const int32_t* token_rows, int64_t total_rows, void* q,
                                          void* scales, void* stream);

/*
 * mxfp4_moe_quantize_scatter with the scale bytes written in the interleaved
 * layout of include/mxfp4.h (scales_il [k/512, total_rows, 16]), the A operand
 * of mxfp4_grouped_gemm_nt_interleaved; codes, and which rows are written, as
 * mxfp4_moe_quantize_scatter.  k a positive multiple of 512 and
 * total_rows * k / 32 < 2^31 (MXFP4_ERR_INVALID_ARG otherwise); other limits as
 * above.
 */
mxfp4_status_t mxfp4_moe_quantize_scatter_interleaved(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                                      const int32_t* token_rows, int64_t total_rows, void* q,
                                                      void* scales_il, void* stream);

/*
 * The same with MXFP8 rows (mxfp8.h's format: q8 [total_rows, k] E4M3 codes,
 * 8-byte aligned), for the W4A8 grouped GEMM.
 */
mxfp4_status_t mxfp8_moe_quantize_scatter(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                          const int32_t* token_rows, int64_t total_rows, void* q8,
                                          void* scales, void* stream);

/* mxfp8_moe_quantize_scatter with the scale bytes interleaved (scales_il
 * [k/512, total_rows, 16]), the A operand of
 * mxfp8_grouped_gemm_w4a8_nt_interleaved; limits as for
 * mxfp4_moe_quantize_scatter_interleaved. */
mxfp4_status_t mxfp8_moe_quantize_scatter_interleaved(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                                      const int32_t* token_rows, int64_t total_rows, void* q8,
                                                      void* scales_il, void* stream);

/*
 * Weighted combine: out[t, :] = sum over slots j in order 0..top_k-1 whose row
 * r = token_rows[t, j] lies in [0, total_rows) of topk_weights[t, j] *
 * y[r, :], as fp32 fused multiply-adds from 0; out is BF16 (nearest-even) or
 * fp32 by out_type.  A token with no kept slot gets zeros.
 *   y_bf16 [total_rows, n] (the grouped GEMM's BF16 output, 2-byte aligned);
 *   out [tokens, n] (2- or 4-byte aligned).  With n % 8 == 0 and 16-byte
 *   aligned y and out, rows move in 16-byte pieces.
 * Limits: 0 <= n <= 2^30, 1 <= top_k <= 256, 0 <= total_rows < 2^31,
 * tokens * ceil(n / 8) < 2^31.  tokens == 0 or n == 0 is a no-op.
 */
mxfp4_status_t mxfp4_moe_combine(const void* y_bf16, int64_t total_rows, int64_t n, const int32_t* token_rows,
                                 const float* topk_weights, int64_t tokens, int32_t top_k, void* out,
                                 mxfp4_out_t out_type, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_MOE_H_ */
