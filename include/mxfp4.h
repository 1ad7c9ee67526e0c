/*
 * mxfp4.h - C ABI of the MI355X (gfx950) MXFP4 quantize / GEMM library.
 *
 * Formats (the "Packed MXFP4 & NVFP4 GEMM + mega-MoE (SM100, true 2-CTA
 * multicast)" page, Summary; the "fp4_quantization" Mojo module page,
 * quantize_dynamic_block_scaled_mxfp4 and matmul_dynamic_block_scaled_mxfp4):
 *   - an MXFP4 operand of `rows` x `k` elements is a pair of row-major byte
 *     arrays, K innermost:
 *       q      uint8 [rows, k/2]   E2M1 codes, element 2j in the low nibble
 *                                  of byte j, element 2j+1 in the high nibble;
 *       scales uint8 [rows, k/32]  one E8M0 byte per 32 consecutive elements
 *                                  of a row (byte b means 2^(b-127)).
 *   - E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
 *     magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *
 * Conventions shared by every entry point:
 *   - All buffer pointers are device pointers on the calling thread's current
 *     HIP device.  Buffers are owned by the caller; the library never frees,
 *     keeps or allocates memory on these paths.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous: they enqueue kernels and return without
 *     synchronising, so they may be captured into a HIP graph.
 *   - All arguments are checked on the host before anything is launched; a
 *     failed check returns a non-OK status and launches nothing.  Sizes are
 *     elements, not bytes.  Alignment: BF16 inputs, code arrays (q, a_q, b_q),
 *     outputs (c) and workspaces 16 bytes, except the quantizer's q output
 *     (4 bytes); scale arrays read by the GEMMs 4 bytes when k % 128 == 0,
 *     otherwise any; the quantizer's scale output any; offsets 4 bytes.  A row
 *     slice of a row-major operand therefore stays valid.
 *   - A zero-sized problem (rows, m, n or total_m equal to 0) is a valid no-op.
 *     Limits: m, n, total_m <= 2^30; k <= 2^24 (the tile kernels address a
 *     tile's rows with 32-bit offsets); quantizer rows * k <= 2^40.  A GEMM
 *     whose grid would exceed one launch (2^32 - 1 threads; only outputs far
 *     larger than device memory come near it) returns MXFP4_ERR_HIP and
 *     launches nothing.
 *   - No call aborts or throws; mxfp4_last_error() gives a thread-local text
 *     describing the last non-OK status.
 *   - Calls are reentrant; the only global state is a per-device cache of
 *     device properties filled on first use.
 */
#ifndef MXFP4_H_
#define MXFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP4_ABI_VERSION 1

typedef enum {
  MXFP4_OK = 0,
  MXFP4_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, bad enum */
  MXFP4_ERR_UNSUPPORTED = 2,   /* the current device is not gfx950 */
  MXFP4_ERR_WORKSPACE = 3,     /* workspace smaller than the size query returned */
  MXFP4_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} mxfp4_status_t;

typedef enum {
  MXFP4_OUT_BF16 = 0,          /* C is bfloat16, rounded to nearest-even from fp32 */
  MXFP4_OUT_F32 = 1            /* C is float32 (the fp32 accumulator, unrounded) */
} mxfp4_out_t;

/* ABI version of the loaded library (MXFP4_ABI_VERSION it was built with). */
int mxfp4_abi_version(void);

/* Text for a status code (static storage). */
const char* mxfp4_status_string(mxfp4_status_t status);

/* Thread-local detail for the last non-OK status returned on this thread. */
const char* mxfp4_last_error(void);

/*
 * Dynamic block-scaled quantization BF16 -> MXFP4 ("fp4_quantization" page,
 * quantize_dynamic_block_scaled_mxfp4: BF16 elements to packed MXFP4 with
 * E8M0 block scales; the quadbit README, Accuracy: per-32 single-level
 * activation quantization with an amax recipe).
 *
 * For each row and each 32-element block x[0..31] along K:
 *   amax = max |x_i|;
 *   e = floor(log2 amax) - 2 (the exponent of E2M1's largest value 6 is 2),
 *       e = -127 for amax == 0, clamped to [-127, 127];
 *   scales byte = e + 127;
 *   code_i = sign(x_i) | nearest E2M1 magnitude of |x_i| / 2^e, ties to the
 *            even code, values above 6 saturated to 6; the sign bit is kept
 *            for zero results (-0 and small negatives give code 8).
 *
 *   x_bf16 : bfloat16 [rows, k], row-major (read only)
 *   q      : uint8 [rows, k/2]   (written)
 *   scales : uint8 [rows, k/32]  (written)
 *   k      : > 0, a multiple of 32, at most 2^24
 * NaN or Inf inputs give unspecified codes (the format has no encoding for
 * them); every finite input is encoded exactly as above.
 */
mxfp4_status_t mxfp4_quantize(const void* x_bf16, int64_t rows, int64_t k,
                              void* q, void* scales, void* stream);

/*
 * Block-scaled NT GEMM on MXFP4 operands ("Packed MXFP4 & NVFP4 GEMM +
 * mega-MoE" page, Summary: mxfp4_gemm_nt, [M,K] @ [N,K].T -> [M,N], BF16 out,
 * both operands packed E2M1 with UE8M0 scales at granularity 32):
 *
 *   C[i][j] = sum over 32-blocks t of 2^(sa[i][t] + sb[j][t] - 254)
 *             * sum_{k in t} e2m1(a[i][k]) * e2m1(b[j][k]),
 *
 * accumulated in fp32 (each 32-block product sum is exact; the order of the
 * fp32 additions across blocks is unspecified).
 *
 *   a_q, a_s : A operand, [m, k/2] and [m, k/32]
 *   b_q, b_s : B operand, [n, k/2] and [n, k/32]
 *   c        : [m, n] row-major, element type `c_type`
 *   k        : > 0, a multiple of 32, at most 2^24
 *   workspace: device scratch of at least mxfp4_gemm_nt_workspace_size(m, n, k)
 *              bytes (may be NULL when that size is 0).  A workspace must be
 *              zero-filled before its first use.  Its first 64 KiB hold
 *              per-tile arrival counters that every call returns to zero; the
 *              rest holds partial sums that need no initialisation.  So a
 *              workspace can be reused by later calls, of any shape, without
 *              clearing.
 *              Calls that share one workspace must be stream-ordered;
 *              concurrent calls on one workspace race.
 */
size_t mxfp4_gemm_nt_workspace_size(int64_t m, int64_t n, int64_t k);

mxfp4_status_t mxfp4_gemm_nt(const void* a_q, const void* a_s,
                             const void* b_q, const void* b_s,
                             void* c, mxfp4_out_t c_type,
                             int64_t m, int64_t n, int64_t k,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped per-expert NT GEMM ("fp4_quantization" page,
 * grouped_matmul_block_scaled_mxfp4: per-expert grouped MXFP4 block-scaled
 * matmul on CDNA4; the quadbit README, distributed MoE paragraph: one launch
 * over routed rows segmented by expert).
 *
 * Rows of A are sorted by group: group g owns rows [offsets[g], offsets[g+1]).
 * For every such row r:  C[r][:] = A[r][:] . B[g]^T, as in mxfp4_gemm_nt.
 *
 *   a_q, a_s  : [total_m, k/2], [total_m, k/32]
 *   b_q, b_s  : [num_groups, n, k/2], [num_groups, n, k/32]
 *   offsets   : DEVICE int32 [num_groups + 1], 0 = offsets[0] <= ... <=
 *               offsets[num_groups] = total_m.  Not readable by the host
 *               without a synchronisation, so it is not validated; the kernel
 *               sanitizes it instead: each offset is clamped into [0, total_m]
 *               and replaced by the running maximum of the clamped offsets up
 *               to it, and group g owns the rows from its sanitized offset to
 *               the next.  Malformed offsets therefore give disjoint, in-range
 *               groups (no row is written twice, no access leaves the
 *               buffers); rows no group owns are not written.  A group with
 *               no rows writes nothing.
 *   c         : [total_m, n], element type `c_type`
 *   k         : > 0, a multiple of 32, at most 2^24
 *   num_groups: 1 .. 1024
 *   workspace : at least mxfp4_grouped_gemm_nt_workspace_size(...) bytes.
 * One kernel launch; nothing depends on host knowledge of the group sizes.
 * Groups averaging 192 rows or more use 256x256 tiles (through the persistent
 * tile loop of MXFP4_KERNEL_PERSISTENT when k % 1024 == 0 and the scale
 * arrays are 16-byte aligned), others 128x128 tiles.  Each group's rows equal
 * mxfp4_gemm_nt_ex on that group's slices with the same tile size, bit for bit.
 */
size_t mxfp4_grouped_gemm_nt_workspace_size(int64_t total_m, int32_t num_groups,
                                            int64_t n, int64_t k);

mxfp4_status_t mxfp4_grouped_gemm_nt(const void* a_q, const void* a_s,
                                     const void* b_q, const void* b_s,
                                     const int32_t* offsets, int32_t num_groups,
                                     int64_t total_m, void* c, mxfp4_out_t c_type,
                                     int64_t n, int64_t k,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Interleaved scale layout for the tile GEMMs (the counterpart on this
 * machine of the "fp4_quantization" page's block_scales_interleave /
 * block_scales_interleave_fp4, which reorder a two-dimensional scale array
 * into the order another GPU's tensor cores consume, and of
 * grouped_quantize_dynamic_scaled_fp4_async, which writes its scales in that
 * order while it quantizes).
 *
 * For an operand of `rows` rows and k % 512 == 0, the scale bytes of the
 * row-major array scales[rows][k/32] are stored as scales_il[k/512][rows][16]:
 *
 *   scales_il[(kb / 16) * rows * 16 + r * 16 + kb % 16] = scales[r * k/32 + kb]
 *
 * so the sixteen scale bytes that cover one 512-wide K slab of a row sit next
 * to the next row's.  The GEMM kernels copy a slab's scales of 64 rows with
 * one 1 KB read instead of 64 reads of 16 bytes, each from its own cache line.
 * The values are those of the row-major array: results are bit-identical to
 * the row-major entry points'.  A grouped weight [num_groups, n, k/32] is
 * interleaved per group: [num_groups][k/512][n][16].
 *
 * mxfp4_scales_interleave: scales [groups, rows, k/32] -> scales_il
 *   [groups, k/512, rows, 16] (weights quantized once, offline).  Both arrays
 *   16-byte aligned, not overlapping.  k a positive multiple of 512, at most
 *   2^24; groups * rows * k <= 2^40.  groups == 0 or rows == 0 is a no-op.
 * mxfp4_quantize_interleaved: mxfp4_quantize with the scales written
 *   interleaved (codes as mxfp4_quantize).  k % 512 == 0 and
 *   rows * k / 32 < 2^31.
 * mxfp4_gemm_nt_interleaved: mxfp4_gemm_nt with both scale arrays
 *   interleaved (A over its m rows, B over its n rows), always on the tile
 *   kernels (256 x 256 tiles once they number at least the compute units,
 *   else 128 x 128; mxfp4_gemm_nt_ex with MXFP4_KERNEL_TILE256 / TILE128 on
 *   the row-major arrays gives the same bits).  No workspace.
 * mxfp4_grouped_gemm_nt_interleaved: mxfp4_grouped_gemm_nt with a_s_il over
 *   total_m rows and b_s_il interleaved per group; same kernels, offsets
 *   handling and bits.  No workspace.
 * For the GEMMs: k a positive multiple of 512, at most 2^24; m * k / 32 and
 * n * k / 32 (total_m * k / 32 for the grouped A) below 2^31; scale arrays
 * 16-byte aligned; every other argument as for the row-major entry point.
 * Violations return MXFP4_ERR_INVALID_ARG.
 */
mxfp4_status_t mxfp4_scales_interleave(const void* scales, int64_t groups, int64_t rows, int64_t k,
                                       void* scales_il, void* stream);

mxfp4_status_t mxfp4_quantize_interleaved(const void* x_bf16, int64_t rows, int64_t k,
                                          void* q, void* scales_il, void* stream);

mxfp4_status_t mxfp4_gemm_nt_interleaved(const void* a_q, const void* a_s_il,
                                         const void* b_q, const void* b_s_il,
                                         void* c, mxfp4_out_t c_type,
                                         int64_t m, int64_t n, int64_t k, void* stream);

mxfp4_status_t mxfp4_grouped_gemm_nt_interleaved(const void* a_q, const void* a_s_il,
                                                 const void* b_q, const void* b_s_il,
                                                 const int32_t* offsets, int32_t num_groups,
                                                 int64_t total_m, void* c, mxfp4_out_t c_type,
                                                 int64_t n, int64_t k, void* stream);

/*
 * Prepacked weights for the small-M (decode) GEMM.  The same NT GEMM as
 * mxfp4_gemm_nt (the "Packed MXFP4 & NVFP4 GEMM + mega-MoE" page, Summary:
 * mxfp4_gemm_nt; its decode shapes are the small-M case), with B, a weight
 * quantized once ahead of time, stored in a layout that hands every lane of
 * the MFMA its operand bytes in one contiguous 1 KB read per wave.  The result
 * is bit-identical to mxfp4_gemm_nt_ex with MXFP4_KERNEL_STREAM on the
 * unpacked B, for both output types.
 *
 * Layout (the bytes are B's codes and scales, rearranged; rows past n are zero
 * codes with scale byte 0): for each 64-row panel P of B (P = 0 ..
 * ceil(n/64) - 1, rows 64P .. 64P+63) and each 512-element K pair t, in that
 * order,
 *   codes,  16384 bytes: byte w*4096 + u*1024 + l*16 + c (w, u in 0..3,
 *           l in 0..63, c in 0..15, u = 2s + j) is code byte c of row
 *           64P + 32j + (l % 32) at that row's byte 256t + 128s + 32w +
 *           16*(l / 32);
 *   scales,  1024 bytes: byte w*256 + l*4 + (2s + j) is the scale byte of the
 *           same row for the 32-element block 16t + 8s + 2w + l / 32.
 *
 * mxfp4_prepacked_weight_size gives the two array sizes:
 *   code_bytes = ceil(n/64) * 64 * k/2,  scale_bytes = ceil(n/64) * 64 * k/32.
 * k must be a positive multiple of 512 (MXFP4_ERR_INVALID_ARG otherwise).
 */
mxfp4_status_t mxfp4_prepacked_weight_size(int64_t n, int64_t k, int64_t* code_bytes, int64_t* scale_bytes);

/*
 * Rearranges an MXFP4 weight into the prepacked layout.
 *   b_q, b_s   : [n, k/2], [n, k/32] row-major (read only; b_q 16-byte aligned)
 *   bp_q, bp_s : device buffers of code_bytes and scale_bytes (written;
 *                16-byte aligned), owned by the caller
 *   k          : a positive multiple of 512, at most 2^24
 */
mxfp4_status_t mxfp4_prepack_weight(const void* b_q, const void* b_s, int64_t n, int64_t k,
                                    void* bp_q, void* bp_s, void* stream);

/*
 * C[m, n] = A . B^T with B prepacked (above).  a_q, a_s: A as in
 * mxfp4_gemm_nt, both 16-byte aligned; c: [m, n] row-major of type `c_type`,
 * 16-byte aligned; k a positive multiple of 512.  No workspace.  Built for
 * m up to 128 (one workgroup per 64 columns per 128 rows of A); larger m is
 * computed correctly by more row tiles that each stream the weight again.
 */
mxfp4_status_t mxfp4_gemm_nt_prepacked(const void* a_q, const void* a_s, const void* bp_q, const void* bp_s,
                                       void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * Quantization (as mxfp4_quantize, bit for bit) written straight into the
 * prepacked layout above, for an activation that feeds
 * mxfp4_gemm_nt_prepacked_ab.  x_bf16: [rows, k] row-major, 16-byte aligned;
 * ap_q, ap_s: code_bytes and scale_bytes of mxfp4_prepacked_weight_size(rows,
 * k) (ap_q 16-byte aligned), every byte written (rows up to the next multiple
 * of 64 as zero blocks); k a positive multiple of 512.
 */
mxfp4_status_t mxfp4_quantize_prepacked(const void* x_bf16, int64_t rows, int64_t k, void* ap_q, void* ap_s,
                                        void* stream);

/*
 * C[m, n] = A . B^T with BOTH operands prepacked: ap_q / ap_s are A [m, k]
 * rearranged by mxfp4_prepack_weight (the layout is defined for any [rows, k]
 * MXFP4 operand; rows past m are zero), bp_q / bp_s as above.  Each wave then
 * loads A and B straight into registers and the main loop uses no LDS.  Same
 * result, bit for bit, as mxfp4_gemm_nt_prepacked.  Alignment, k and output
 * as for mxfp4_gemm_nt_prepacked.
 */
mxfp4_status_t mxfp4_gemm_nt_prepacked_ab(const void* ap_q, const void* ap_s, const void* bp_q, const void* bp_s,
                                          void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * mxfp4_gemm_nt_prepacked_ab with K split over workgroups, for shapes with
 * fewer 64-column output panels than compute units (the decode down
 * projection, n = 4096: 64 panels).  The same GEMM ("Packed MXFP4 & NVFP4
 * GEMM + mega-MoE" page, Summary: mxfp4_gemm_nt at its decode shapes; the
 * quadbit README's serving section splits the down projection's K over more
 * CTAs with an fp32 reduction to fill the machine).
 *   splits    : 0 = automatic (enough K ranges to give most compute units a
 *               workgroup, each at least 1024 K long; 1 when the panels
 *               already fill the chip), 1 = no split (exactly
 *               mxfp4_gemm_nt_prepacked_ab), else 2..16 requested ranges of
 *               ceil(pairs / splits) 512-K pairs, rounded up to a multiple of
 *               4 pairs when above 4 (so fewer ranges than asked may result,
 *               none empty).  MXFP4_ERR_INVALID_ARG outside 0..16.
 *   workspace : at least mxfp4_gemm_nt_prepacked_ab_workspace_size(m, n, k,
 *               splits) bytes, 16-byte aligned, zero-filled before its first
 *               use; every call leaves its first 64 KiB (the arrival
 *               counters) zero again, so one workspace serves consecutive
 *               stream-ordered calls of any shape.  Calls that may overlap
 *               (other streams) need workspaces of their own.  NULL / 0 when
 *               the size is 0 (MXFP4_ERR_WORKSPACE if too small).
 * Each output is the sum of the ranges' fp32 partial sums in range order
 * (deterministic, not bit-identical to the unsplit kernel), rounded once to
 * the output type.  Split-K needs at most 16384 output tiles (64-column
 * panels x 128-row tiles); MXFP4_ERR_INVALID_ARG beyond.  Other arguments as
 * for mxfp4_gemm_nt_prepacked_ab.
 */
size_t mxfp4_gemm_nt_prepacked_ab_workspace_size(int64_t m, int64_t n, int64_t k, int32_t splits);

mxfp4_status_t mxfp4_gemm_nt_prepacked_ab_ex(const void* ap_q, const void* ap_s, const void* bp_q, const void* bp_s,
                                             void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                                             int32_t splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel selection for tests and tuning.  mxfp4_gemm_nt chooses a kernel per
 * shape; mxfp4_gemm_nt_ex lets a caller force one so every kernel can be
 * checked on any shape.  `kernel` values:
 *   MXFP4_KERNEL_AUTO      the shape-based choice mxfp4_gemm_nt makes
 *   MXFP4_KERNEL_TILE256   256x256 output tiles, LDS-staged scaled MFMA
 *   MXFP4_KERNEL_TILE128   128x128 output tiles (more tiles for mid sizes)
 *   MXFP4_KERNEL_SPLITK    M<=128 bandwidth path, K split `splits` ways with
 *                          an fp32 reduction in the workspace
 *   MXFP4_KERNEL_STREAM    small-M weight-streaming path: 64-column tiles over
 *                          the whole K, operands copied into LDS in 512-K
 *                          units; needs k % 512 == 0 and 16-byte aligned
 *                          scale arrays (MXFP4_ERR_INVALID_ARG otherwise)
 *   MXFP4_KERNEL_PERSISTENT 256x256 tiles as TILE256, one workgroup per compute
 *                          unit looping over its tiles and loading the next
 *                          tile's first K stage during a tile's epilogue;
 *                          results identical to TILE256; needs k % 1024 == 0
 *                          and 16-byte aligned scale arrays
 *                          (MXFP4_ERR_INVALID_ARG otherwise)
 * `splits` is only read for MXFP4_KERNEL_SPLITK (0 = automatic, else 1..64).
 * For m <= 128 the automatic choice is MXFP4_KERNEL_STREAM when its
 * requirements hold, else MXFP4_KERNEL_SPLITK; neither needs a workspace then.
 * The workspace needed is mxfp4_gemm_nt_ex_workspace_size(...).
 */
typedef enum {
  MXFP4_KERNEL_AUTO = 0,
  MXFP4_KERNEL_TILE256 = 1,
  MXFP4_KERNEL_TILE128 = 2,
  MXFP4_KERNEL_SPLITK = 3,
  MXFP4_KERNEL_STREAM = 4,
  MXFP4_KERNEL_PERSISTENT = 5
} mxfp4_kernel_t;

size_t mxfp4_gemm_nt_ex_workspace_size(int64_t m, int64_t n, int64_t k,
                                       mxfp4_kernel_t kernel, int32_t splits);

mxfp4_status_t mxfp4_gemm_nt_ex(const void* a_q, const void* a_s,
                                const void* b_q, const void* b_s,
                                void* c, mxfp4_out_t c_type,
                                int64_t m, int64_t n, int64_t k,
                                mxfp4_kernel_t kernel, int32_t splits,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxfp4_gemm_nt_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results as mxfp4_gemm_nt_ex (bit for bit), with
 * no workspace argument: the split-K partial sums and arrival counters
 * (MXFP4_KERNEL_SPLITK with splits > 1, the only choice that needs a
 * workspace) live in a library-owned static device array of
 * MXFP4_NOALLOC_SCRATCH_BYTES bytes, one on each GPU the library runs on,
 * held until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); on its first call on a device it
 * looks up that device's copy of the array (with the device current) and
 * keeps the address.  A call whose workspace
 * (mxfp4_gemm_nt_ex_workspace_size) exceeds the array returns
 * MXFP4_ERR_WORKSPACE and launches nothing.  The array keeps the last call's
 * contents; each split-K call first zeroes the counters with a small kernel
 * on `stream`.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (on different streams, or from several threads)
 * race on it and must be serialized by the caller.
 */
#define MXFP4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

mxfp4_status_t mxfp4_gemm_nt_ex_noalloc(const void* a_q, const void* a_s,
                                        const void* b_q, const void* b_s,
                                        void* c, mxfp4_out_t c_type,
                                        int64_t m, int64_t n, int64_t k,
                                        mxfp4_kernel_t kernel, int32_t splits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H_ */
