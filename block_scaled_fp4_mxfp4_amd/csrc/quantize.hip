// BF16 -> MXFP4 dynamic block quantization for gfx950.
//
// Operation ("fp4_quantization" Mojo module page, Functions,
// quantize_dynamic_block_scaled_mxfp4): per 32-element block, amax -> shared exponent e = floor(log2 amax) - 2 clamped
// to the E8M0 range -> each element x / 2^e rounded to nearest-even E2M1 with
// saturation at 6, two codes per byte (element 2j in the low nibble).
//
// Layout: because K is a multiple of 32 and all three arrays are row-major, the
// rows x K input is a flat sequence of blocks; block b reads bytes [64b, 64b+64)
// of x, writes bytes [16b, 16b+16) of q and byte b of the scales.  With
// interleaved scales (k % 512 == 0, the tile GEMMs' copy layout
// [k/512, rows, 16]) the blocks are walked in the order of that layout
// instead: step b is block 16 g + b % 16 of row r, where b / 16 = g * rows + r,
// and writes scale byte b.  Each wave still reads one 1 KB run of x (the 16
// blocks of one 512-wide slab of a row), and each 128-byte line of scales is
// written by neighbouring waves: walked in row order, a line of the
// interleaved layout would collect the pieces of 8 rows from workgroups on
// different XCDs, each writing back its part of the line.
//
// Mapping: 4 lanes per block, 16 bytes (8 BF16) per lane, so one wave64 covers
// 16 blocks with 1 KiB of fully coalesced loads.  HBM-bound: 2.53125 bytes per
// element (2 in, 0.5 + 1/32 out).
//
// Arithmetic:
//  * amax is an integer max over the BF16 magnitude bits (x & 0x7FFF): for
//    non-negative finite floats bit order equals value order.
//  * floor(log2 amax) = E - 127 for a normal amax with biased exponent E, so the
//    scale byte is e + 127 = E - 2.  Every amax below 2^-125 (E <= 2, including
//    subnormals and zero) lands on the lower clamp e = -127, byte 0.  Finite
//    BF16 has E <= 254, so the byte never exceeds 252 and the upper clamp never
//    applies.  Hence byte = max(E - 2, 0).
//  * The element encoding uses the CDNA4 convert v_cvt_scalef32_pk_fp4_bf16,
//    which divides by the power of two held in the exponent field of its fp32
//    scale operand (only that field is read, so exponent field 0 means 2^-127)
//    and rounds to nearest-even with saturation.  Passing (byte << 23) as the
//    scale's bits therefore applies exactly 2^-e.  That this instruction agrees
//    with the reference encoding for every finite BF16 input and every scale
//    byte was checked exhaustively on the device before it was adopted, and the
//    parity tests re-check it through this kernel.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantUnroll = 2;   // blocks in flight per lane group per iteration (with the grid cap, large
                                   // operands take several iterations, so stores overlap the next loads)

__device__ __forceinline__ uint32_t umax16x2(uint32_t a, uint32_t b) {
  // independent max of the low and high 16-bit halves
  uint32_t lo = max(a & 0xFFFFu, b & 0xFFFFu);
  uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}

// max over the 4 lanes of an aligned quad (DPP quad permutes)
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // lane ^ 1
  v = max(v, o);
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);            // lane ^ 2
  return max(v, o);
}

// IL: interleaved scales; then rows * k/32 < 2^31 (`bpr` = k/32 blocks per
// row, a multiple of 16), so block indices fit 32 bits.
template <bool IL>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(
    const uint4* __restrict__ x, uint32_t* __restrict__ q, uint8_t* __restrict__ scales,
    int64_t nblocks, uint32_t bpr, uint32_t rows) {
  const int lane4 = threadIdx.x & 3;
  const int64_t groups_per_grid = (int64_t)gridDim.x * (kQuantThreads / 4);
  int64_t blk = (int64_t)blockIdx.x * (kQuantThreads / 4) + (threadIdx.x >> 2);

  for (; blk < nblocks; blk += groups_per_grid * kQuantUnroll) {
    uint4 v[kQuantUnroll];
    int64_t src[kQuantUnroll];   // the step's block in x and q (row-major order)
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int64_t b = blk + u * groups_per_grid;
      src[u] = b;
      if constexpr (IL) {
        const uint32_t piece = (uint32_t)b >> 4, g = piece / rows, r = piece - g * rows;
        src[u] = (int64_t)r * bpr + g * 16 + ((uint32_t)b & 15);
      }
      // out-of-range groups load a valid block (block 0) and store nothing
      // BF16 input read once: non-temporal (same-box A/B on 4096 x 4096: 9.73-9.84 vs 9.84-10.19 us)
      const v4i t = __builtin_nontemporal_load((const v4i*)(x + (b < nblocks ? src[u] : 0) * 4 + lane4));
      v[u] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int64_t b = blk + u * groups_per_grid;
      const uint32_t m01 = umax16x2(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu);
      const uint32_t m23 = umax16x2(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu);
      const uint32_t m = umax16x2(m01, m23);
      uint32_t amax_bits = max(m & 0xFFFFu, m >> 16);
      amax_bits = quad_max(amax_bits);
      const int exp_field = (int)(amax_bits >> 7);
      const uint32_t sbyte = (uint32_t)max(exp_field - 2, 0);
      const float scale = __uint_as_float(sbyte << 23);
      uint32_t packed = 0;
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v[u].x), scale, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v[u].y), scale, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v[u].z), scale, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v[u].w), scale, 3);
      if (b < nblocks) {
        q[src[u] * 4 + lane4] = packed;
        if (lane4 == 0) scales[b] = (uint8_t)sbyte;
      }
    }
  }
}

// Scale bytes [groups, rows, k/32] -> interleaved [groups, k/512, rows, 16]:
// one 16-byte piece per thread, in the output's order (coalesced stores).
__global__ __launch_bounds__(256) void scales_interleave_kernel(const uint4* __restrict__ src,
                                                                uint4* __restrict__ dst, int64_t pieces,
                                                                int64_t rows, int64_t gpr) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < pieces; d += stride) {
    // d = (e * gpr + g) * rows + r  <-  source piece (e * rows + r) * gpr + g
    const int64_t eg = d / rows, r = d - eg * rows;
    const int64_t e = eg / gpr, g = eg - e * gpr;
    dst[d] = src[(e * rows + r) * gpr + g];
  }
}

// ---------------------------------------------------------------------------
// The same quantization written straight into the prepacked operand layout of
// the small-M GEMM (include/mxfp4.h, mxfp4_prepack_weight): per 64-row panel
// P and 512-K pair t, a block's 16 code bytes form one lane's operand, at
//   (P * pairs + t) * 16384 + w * 4096 + (2s + j) * 1024 + l * 16,
// and its scale byte sits at (P * pairs + t) * 1024 + w * 256 + l * 4 + 2s + j,
// where for row r and 32-element block kb of that row: j = (r % 64) / 32,
// t = kb / 16, s = (kb / 8) % 2, w = (kb / 2) % 4, l = r % 32 + 32 * (kb % 2).
// Rows from `rows` up to the panel boundary are written as zero blocks (code
// 0, scale byte 0: what a zero row quantizes to).  Codes and scale bytes are
// those of quantize_kernel, bit for bit; only where they are stored differs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kQuantThreads) void quantize_prepacked_kernel(
    const uint4* __restrict__ x, uint32_t* __restrict__ q, uint8_t* __restrict__ scales, int64_t rows,
    int kblocks, int64_t nblocks) {
  const int lane4 = threadIdx.x & 3;
  const int64_t groups_per_grid = (int64_t)gridDim.x * (kQuantThreads / 4);
  const int pairs = kblocks / 16;
  for (int64_t b = (int64_t)blockIdx.x * (kQuantThreads / 4) + (threadIdx.x >> 2); b < nblocks;
       b += groups_per_grid) {
    const int64_t r = b / kblocks;
    const int kb = (int)(b - r * kblocks);
    uint4 v = {0u, 0u, 0u, 0u};
    if (r < rows) v = x[b * 4 + lane4];   // padded rows past `rows` encode a zero block
    const uint32_t m01 = umax16x2(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu);
    const uint32_t m23 = umax16x2(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu);
    const uint32_t m = umax16x2(m01, m23);
    uint32_t amax_bits = max(m & 0xFFFFu, m >> 16);
    amax_bits = quad_max(amax_bits);
    const uint32_t sbyte = (uint32_t)max((int)(amax_bits >> 7) - 2, 0);
    const float scale = __uint_as_float(sbyte << 23);
    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v.x), scale, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v.y), scale, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v.z), scale, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, v.w), scale, 3);
    int64_t word, sidx;
    prepacked_index(r, kb, pairs, word, sidx);
    q[word + lane4] = packed;
    if (lane4 == 0) scales[sidx] = (uint8_t)sbyte;
  }
}

// ---------------------------------------------------------------------------
// BF16 -> MXFP8 (E4M3 elements, E8M0 scales): the activation format of the W4A8
// GEMM ("fp4_quantization" page, quantize_dynamic_scaled_fp4fp8: BF16 to
// NVFP4 / MXFP4 / MXFP8 with per-block scale factors).  Same block mapping as
// above; each lane writes its 8 elements as 8 code bytes.
//  * e = floor(log2 amax) - 8 (E4M3's largest exponent is 8), clamped to the
//    E8M0 range: byte = max(E - 8, 0) for amax's biased exponent E.
//  * Elements: x / 2^e rounded to nearest-even E4M3, magnitudes above 448
//    saturating to 448.  Every magnitude is first clamped to 448 * 2^e, which
//    BF16 represents exactly (exponent field 8 + byte, mantissa 0x60): values
//    in (448, 464] * 2^e round to 448 anyway and larger ones saturate there,
//    so after the clamp the convert only ever sees in-range values and the
//    result does not depend on its overflow handling.  The scaled convert
//    v_cvt_scalef32_pk_fp8_bf16 then applies 2^-e from the scale's exponent
//    field and rounds to nearest-even; the parity tests check it against the
//    reference encoding for every finite BF16 value at every scale byte.
// ---------------------------------------------------------------------------

typedef short short2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t clamp_mag16x2(uint32_t w, uint32_t bound) {
  const uint32_t lo = min(w & 0x7FFFu, bound) | (w & 0x8000u);
  const uint32_t hi = min((w >> 16) & 0x7FFFu, bound) | ((w >> 16) & 0x8000u);
  return lo | (hi << 16);
}

__device__ __forceinline__ uint32_t cvt_fp8x4(uint32_t w01, uint32_t w23, float scale) {
  short2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w01), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w23), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// IL: interleaved scales, the blocks walked in that layout's order as in
// quantize_kernel (rows * k/32 < 2^31).
template <bool IL>
__global__ __launch_bounds__(kQuantThreads) void quantize_mxfp8_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, uint8_t* __restrict__ scales, int64_t nblocks,
    uint32_t bpr, uint32_t rows) {
  const int lane4 = threadIdx.x & 3;
  const int64_t groups_per_grid = (int64_t)gridDim.x * (kQuantThreads / 4);
  int64_t blk = (int64_t)blockIdx.x * (kQuantThreads / 4) + (threadIdx.x >> 2);

  for (; blk < nblocks; blk += groups_per_grid * kQuantUnroll) {
    uint4 v[kQuantUnroll];
    int64_t src[kQuantUnroll];   // the step's block in x and q (row-major order)
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int64_t b = blk + u * groups_per_grid;
      src[u] = b;
      if constexpr (IL) {
        const uint32_t piece = (uint32_t)b >> 4, g = piece / rows, r = piece - g * rows;
        src[u] = (int64_t)r * bpr + g * 16 + ((uint32_t)b & 15);
      }
      // BF16 input read once: non-temporal (same-box A/B on 4096 x 4096: 9.73-9.84 vs 9.84-10.19 us)
      const v4i t = __builtin_nontemporal_load((const v4i*)(x + (b < nblocks ? src[u] : 0) * 4 + lane4));
      v[u] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int64_t b = blk + u * groups_per_grid;
      const uint32_t m01 = umax16x2(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu);
      const uint32_t m23 = umax16x2(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu);
      const uint32_t m = umax16x2(m01, m23);
      uint32_t amax_bits = max(m & 0xFFFFu, m >> 16);
      amax_bits = quad_max(amax_bits);
      const int exp_field = (int)(amax_bits >> 7);
      const uint32_t sbyte = (uint32_t)max(exp_field - 8, 0);
      const float scale = __uint_as_float(sbyte << 23);
      const uint32_t bound = ((8u + sbyte) << 7) | 0x60u;      // 448 * 2^e as BF16 magnitude bits
      const uint32_t lo = cvt_fp8x4(clamp_mag16x2(v[u].x, bound), clamp_mag16x2(v[u].y, bound), scale);
      const uint32_t hi = cvt_fp8x4(clamp_mag16x2(v[u].z, bound), clamp_mag16x2(v[u].w, bound), scale);
      if (b < nblocks) {
        q[src[u] * 4 + lane4] = make_uint2(lo, hi);
        if (lane4 == 0) scales[b] = (uint8_t)sbyte;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The MXFP8 quantization written straight into the FP8 prepacked operand
// layout of the W4A8 GEMM on both operands prepacked (include/mxfp8.h).  The
// FP8 operand of the scaled MFMA takes, in lane half h of a 64-K step, the
// 16 codes at K [16h, 16h + 16) in its first four registers and those at
// [32 + 16h, 48 + 16h) in its last four, with the scale byte of the step's
// 32-block h.  Per 64-row panel P and 512-K pair t the layout therefore holds,
// for wave w (the 64-K step w of each 256-K stage s), u = 2s + j (row block j
// of the panel) and register half e, one 1 KB piece of the 64 lanes' 16-byte
// halves:
//   codes (P * pairs + t) * 32768 + w * 8192 + u * 2048 + e * 1024 + l * 16,
// and the scale bytes exactly where the MXFP4 prepacked layout keeps them.
// A lane quad of this kernel quantizes 32-block kb of row r (the step's block
// e = kb % 2); quad lane q holds its K [8q, 8q + 8), which is lane
// l = r % 32 + 32 (q / 2), register half e, bytes [8 (q % 2), 8 (q % 2) + 8).
// Rows from `rows` up to the panel boundary are written as zero blocks.  Codes
// and scale bytes are those of quantize_mxfp8_kernel, bit for bit.
__global__ __launch_bounds__(kQuantThreads) void quantize_mxfp8_prepacked_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ scales, int64_t rows,
    int kblocks, int64_t nblocks) {
  const int lane4 = threadIdx.x & 3;
  const int64_t groups_per_grid = (int64_t)gridDim.x * (kQuantThreads / 4);
  const int pairs = kblocks / 16;
  for (int64_t b = (int64_t)blockIdx.x * (kQuantThreads / 4) + (threadIdx.x >> 2); b < nblocks;
       b += groups_per_grid) {
    const int64_t r = b / kblocks;
    const int kb = (int)(b - r * kblocks);
    uint4 v = {0u, 0u, 0u, 0u};
    if (r < rows) v = x[b * 4 + lane4];   // padded rows past `rows` encode a zero block
    const uint32_t m01 = umax16x2(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu);
    const uint32_t m23 = umax16x2(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu);
    const uint32_t m = umax16x2(m01, m23);
    uint32_t amax_bits = max(m & 0xFFFFu, m >> 16);
    amax_bits = quad_max(amax_bits);
    const uint32_t sbyte = (uint32_t)max((int)(amax_bits >> 7) - 8, 0);
    const float scale = __uint_as_float(sbyte << 23);
    const uint32_t bound = ((8u + sbyte) << 7) | 0x60u;      // 448 * 2^e as BF16 magnitude bits
    const uint32_t lo = cvt_fp8x4(clamp_mag16x2(v.x, bound), clamp_mag16x2(v.y, bound), scale);
    const uint32_t hi = cvt_fp8x4(clamp_mag16x2(v.z, bound), clamp_mag16x2(v.w, bound), scale);
    int64_t word, sidx;
    prepacked_index(r, kb, pairs, word, sidx);   // the scale byte's place (the code word's is FP4's)
    const int64_t panel = r / 64;
    const int rr = (int)(r - panel * 64);
    const int j = rr >> 5, t = kb >> 4, s = (kb >> 3) & 1, w = (kb >> 1) & 3, e = kb & 1;
    const int l = (rr & 31) + 32 * (lane4 >> 1);
    const int64_t off = (panel * pairs + t) * 32768 + w * 8192 + (2 * s + j) * 2048 + e * 1024 + l * 16 +
                        8 * (lane4 & 1);
    *(uint2*)(q + off) = make_uint2(lo, hi);
    if (lane4 == 0) scales[sidx] = (uint8_t)sbyte;
  }
}

}  // namespace

hipError_t launch_quantize_mxfp8(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                                 hipStream_t stream, int num_cus, bool interleaved) {
  const int64_t nblocks = rows * (k / 32);
  if (interleaved && (k % 512 != 0 || nblocks >= ((int64_t)1 << 31))) return hipErrorInvalidValue;
  const int64_t groups_needed = (nblocks + kQuantUnroll - 1) / kQuantUnroll;
  int64_t grid = (groups_needed + (kQuantThreads / 4) - 1) / (kQuantThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  const auto kernel = interleaved ? quantize_mxfp8_kernel<true> : quantize_mxfp8_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream, (const uint4*)x, (uint2*)q,
                     (uint8_t*)scales, nblocks, (uint32_t)(k / 32), (uint32_t)rows);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                           hipStream_t stream, int num_cus, bool interleaved) {
  const int64_t nblocks = rows * (k / 32);
  if (interleaved && (k % 512 != 0 || nblocks >= ((int64_t)1 << 31))) return hipErrorInvalidValue;
  const int64_t groups_needed = (nblocks + kQuantUnroll - 1) / kQuantUnroll;
  int64_t grid = (groups_needed + (kQuantThreads / 4) - 1) / (kQuantThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  if (interleaved)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream,
                       (const uint4*)x, (uint32_t*)q, (uint8_t*)scales, nblocks, (uint32_t)(k / 32), (uint32_t)rows);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream,
                       (const uint4*)x, (uint32_t*)q, (uint8_t*)scales, nblocks, (uint32_t)(k / 32), (uint32_t)rows);
  return hipGetLastError();
}

hipError_t launch_scales_interleave(const void* scales, int64_t groups, int64_t rows, int64_t k, void* out,
                                    hipStream_t stream, int num_cus) {
  if (k % 512 != 0 || groups < 1 || rows < 1) return hipErrorInvalidValue;
  const int64_t gpr = k / 512, pieces = groups * rows * gpr;
  int64_t grid = (pieces + 255) / 256;
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  hipLaunchKernelGGL(scales_interleave_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (const uint4*)scales,
                     (uint4*)out, pieces, rows, gpr);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_prepacked(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                                           hipStream_t stream, int num_cus) {
  const int64_t padded = (rows + 63) / 64 * 64;
  const int64_t nblocks = padded * (k / 32);
  int64_t grid = (nblocks + (kQuantThreads / 4) - 1) / (kQuantThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(quantize_mxfp8_prepacked_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream,
                     (const uint4*)x, (uint8_t*)q, (uint8_t*)scales, rows, (int)(k / 32), nblocks);
  return hipGetLastError();
}

hipError_t launch_quantize_prepacked(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                                     hipStream_t stream, int num_cus) {
  const int64_t padded = (rows + 63) / 64 * 64;
  const int64_t nblocks = padded * (k / 32);
  int64_t grid = (nblocks + (kQuantThreads / 4) - 1) / (kQuantThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(quantize_prepacked_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream,
                     (const uint4*)x, (uint32_t*)q, (uint8_t*)scales, rows, (int)(k / 32), nblocks);
  return hipGetLastError();
}

}  // namespace mxfp4
