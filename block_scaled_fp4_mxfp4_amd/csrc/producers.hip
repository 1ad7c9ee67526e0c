// Fused producers that emit MXFP4 activations (gfx950).
//
// The quadbit README ("Accuracy (real models)", "The stack") runs its FP4
// transformer block with fused RMSNorm, residual-add and SwiGLU quantizers
// around the GEMMs: the kernel that produces an activation writes it already
// quantized, so the BF16 activation never makes a round trip through HBM
// before the quantizer reads it.  Two producers:
//
//  rmsnorm_quantize_kernel: one workgroup per row.  Each thread holds 2, 4 or
//    16 chunks of 8 consecutive elements in registers (k <= 32768).
//    h = RNE_bf16(x + residual) (fp32 add: exact for BF16 inputs unless their
//    exponents differ by more than 15, where the smaller one lies far below any
//    BF16 rounding midpoint, so the result equals the rounding of the exact sum);
//    the row's sum of squares in fp64 (each square exact), a fixed-order
//    wave/workgroup reduction, inv = 1 / sqrt(sum / k + eps) in fp64, then
//    y = RNE_bf16((h * inv) * gamma) from fp64 with a single rounding.  The
//    fp64 path makes y equal to the nearest BF16 of the exact value except
//    where that value lies within ~2^-50 of a BF16 rounding midpoint.
//  swiglu_quantize_kernel: elementwise y = RNE_bf16(g * u / (1 + exp(-g))) in
//    fp32 with the hardware exp2 and reciprocal (the accurate library expf and
//    IEEE divide cost about 30 instructions per element, which made the kernel
//    ALU-bound) over the flat 32-element blocks of the [rows, k] output, gate
//    and up read with a row stride (so one [rows, 2k] gate|up buffer serves).
//
// Both quantize y exactly as the MXFP4 quantizer does (4 lanes per 32-element
// block, integer amax, scale byte max(E - 2, 0), the CDNA4 scaled FP4 convert)
// and can also store y itself.  HBM-bound.
//
// PREPACKED: the same code and scale bytes stored in the prepacked operand
// layout of the decode GEMM (include/mxfp4.h), so the activation's producer
// hands the small-M GEMM its operand with no quantization launch in between
// (rows up to the next multiple of 64 are written as zero blocks, as the
// prepacked quantizer writes them).
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kNormThreads = 256;
constexpr int kProdThreads = 256;
constexpr int kProdUnroll = 2;

__device__ __forceinline__ uint32_t umax16x2(uint32_t a, uint32_t b) {
  return max(a & 0xFFFFu, b & 0xFFFFu) | (max(a >> 16, b >> 16) << 16);
}

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // lane ^ 1
  v = max(v, o);
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);            // lane ^ 2
  return max(v, o);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp64 -> BF16 bits with a single nearest-even rounding.  The producers' values
// are far inside fp64's normal range, so only BF16's own ranges matter:
// normals keep 7 of the 52 mantissa bits (the rounding carry may step the
// exponent), below 2^-126 the BF16 quantum is 2^-133, beyond the largest BF16
// value the result is infinity.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const uint64_t bits = (uint64_t)__double_as_longlong(d);
  const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
  uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return sign;
  const int e = (int)(mag >> 52) - 1023;
  if (e >= -126) {
    mag += (((uint64_t)1 << 44) - 1) + ((mag >> 45) & 1);
    const int e2 = (int)(mag >> 52) - 1023;
    if (e2 > 127) return sign | 0x7F80u;
    return sign | (uint32_t)((e2 + 127) << 7) | (uint32_t)((mag >> 45) & 0x7F);
  }
  const double n = rint(fabs(d) * 0x1p133);   // exact scaling; at most 128 (the smallest normal's bits)
  return sign | (uint32_t)n;
}

__device__ __attribute__((noinline)) uint32_t f64_to_bf16_rne_slow(double d) { return f64_to_bf16_rne(d); }

// f64_to_bf16_rne through the hardware conversions: d -> fp32 (nearest even)
// -> BF16 (nearest even).  The first rounding never steps over an fp32 value,
// and every BF16 midpoint is one, so the two agree with the direct rounding
// unless the fp32 value lands exactly on a midpoint (its last 16 bits 0x8000)
// or is subnormal, zero, at or above 2^127, or not finite: those take the
// direct path.
__device__ __forceinline__ uint32_t f64_to_bf16_rne_fast(double d) {
  const uint32_t b = __float_as_uint((float)d);
  const uint32_t ex = (b >> 23) & 0xFFu;
  if (__builtin_expect(ex >= 1u && ex <= 253u && (b & 0xFFFFu) != 0x8000u, 1))
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return f64_to_bf16_rne_slow(d);
}

// 8 BF16 codes -> packed E2M1 word and the block's scale byte (quad-wide amax)
__device__ __forceinline__ uint32_t quantize8(const uint4& v, uint32_t& sbyte) {
  const uint32_t m = umax16x2(umax16x2(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                              umax16x2(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
  const uint32_t amax_bits = quad_max(max(m & 0xFFFFu, m >> 16));
  sbyte = (uint32_t)max((int)(amax_bits >> 7) - 2, 0);
  const float scale = __uint_as_float(sbyte << 23);
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, v.x), scale, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, v.y), scale, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, v.z), scale, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, v.w), scale, 3);
  return p;
}

__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  return pack_bf16x2(bf16_lo(a) + bf16_lo(b), bf16_hi(a) + bf16_hi(b));
}

__device__ __forceinline__ double sumsq_bf16x2(uint32_t w, double acc) {
  const double lo = bf16_lo(w), hi = bf16_hi(w);
  return fma(hi, hi, fma(lo, lo, acc));
}

// LAYOUT: where the MXFP4 bytes go (ProducerLayout in launch.hpp): row-major,
// the prepacked operand layout, or row-major codes with interleaved scales
// ([k/512, rows, 16], the tile GEMMs' copy layout; rows * k/32 < 2^31).
template <bool HAS_RES, int SLOTS, int LAYOUT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_quantize_kernel(
    // x, res, h_out and y_out may share memory (in-place residual and output): no __restrict__ on them
    const uint4* x, const uint4* res, const uint4* __restrict__ gamma, float eps, int rows, int k,
    uint4* h_out, uint4* y_out, uint32_t* __restrict__ q, uint8_t* __restrict__ scales) {
  __shared__ double red[kNormThreads / 64];
  constexpr bool PREPACKED = LAYOUT == kLayoutPrepacked;
  const int chunks = k >> 3;                         // 8 elements (one uint4) per chunk
  const int64_t rbase = (int64_t)blockIdx.x * chunks;
  if (PREPACKED && (int)blockIdx.x >= rows) {
    // a padding row of the last 64-row panel: zero codes and scale bytes
    for (int c = threadIdx.x; c < chunks; c += kNormThreads) {
      int64_t word, sidx;
      prepacked_index(blockIdx.x, c >> 2, k / 512, word, sidx);
      q[word + (c & 3)] = 0u;
      if ((c & 3) == 0) scales[sidx] = 0;
    }
    return;
  }
  uint4 h[SLOTS], gm[SLOTS];
  double ss = 0.0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int c = s * kNormThreads + threadIdx.x;
    h[s] = make_uint4(0u, 0u, 0u, 0u);
    gm[s] = make_uint4(0u, 0u, 0u, 0u);
    if (c < chunks) {
      h[s] = x[rbase + c];
      gm[s] = gamma[c];   // loaded with the row, so the second phase waits on nothing
    }
  }
  if (HAS_RES) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int c = s * kNormThreads + threadIdx.x;
      if (c < chunks) {
        const uint4 r = res[rbase + c];
        h[s] = make_uint4(add_bf16x2(h[s].x, r.x), add_bf16x2(h[s].y, r.y), add_bf16x2(h[s].z, r.z),
                          add_bf16x2(h[s].w, r.w));
        if (h_out) h_out[rbase + c] = h[s];
      }
    }
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s)
    ss = sumsq_bf16x2(h[s].w, sumsq_bf16x2(h[s].z, sumsq_bf16x2(h[s].y, sumsq_bf16x2(h[s].x, ss))));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double total = ((red[0] + red[1]) + red[2]) + red[3];
  const double inv = 1.0 / sqrt(total / (double)k + (double)eps);

#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int c = s * kNormThreads + threadIdx.x;
    if (c >= chunks) continue;   // uniform over each lane quad (chunks % 4 == 0)
    const uint4 g = gm[s];
    const uint32_t hw[4] = {h[s].x, h[s].y, h[s].z, h[s].w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t yw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = f64_to_bf16_rne_fast((double)bf16_lo(hw[i]) * inv * (double)bf16_lo(gw[i]));
      const uint32_t hi = f64_to_bf16_rne_fast((double)bf16_hi(hw[i]) * inv * (double)bf16_hi(gw[i]));
      yw[i] = lo | (hi << 16);
    }
    const uint4 y = make_uint4(yw[0], yw[1], yw[2], yw[3]);
    if (y_out) y_out[rbase + c] = y;
    uint32_t sbyte;
    const uint32_t codes = quantize8(y, sbyte);
    if (PREPACKED) {
      int64_t word, sidx;
      prepacked_index(blockIdx.x, c >> 2, k / 512, word, sidx);
      q[word + (threadIdx.x & 3)] = codes;
      if ((threadIdx.x & 3) == 0) scales[sidx] = (uint8_t)sbyte;
    } else {
      q[rbase + c] = codes;
      if ((threadIdx.x & 3) == 0) {
        if (LAYOUT == kLayoutInterleaved) {   // piece kb / 16 of this row in slab-major order
          const uint32_t kb = (uint32_t)c >> 2;
          scales[(kb >> 4) * (uint32_t)rows * 16 + blockIdx.x * 16 + (kb & 15)] = (uint8_t)sbyte;
        } else {
          scales[(rbase + c) >> 2] = (uint8_t)sbyte;
        }
      }
    }
  }
}

// silu(g) * u with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32,
// each about 1 ulp): exp(-g) = exp2(-g * log2 e).  Relative error at most
// about (|g| + 6) * 2^-24: the product -g * log2 e rounds by |g| * 2^-24 in the
// exponent, exp2 and rcp add an ulp each, 1 + t and the final product half an
// ulp each.  Very negative g gives exp2 = inf, rcp = 0 and a signed zero; very
// positive g gives t = 0 and y = g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float t = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return (g * u) * __builtin_amdgcn_rcpf(1.0f + t);
}

__device__ __forceinline__ uint32_t swiglu_bf16x2(uint32_t g, uint32_t u) {
  return pack_bf16x2(silu_mul(bf16_lo(g), bf16_lo(u)), silu_mul(bf16_hi(g), bf16_hi(u)));
}

// nblocks counts the 32-blocks of `rows` rows, or with the prepacked layout of
// the rows rounded up to 64 (blocks of padding rows are written as zero
// blocks).  With interleaved scales the walk stays row-major (the reads of
// gate and up run along the rows) and each scale byte goes to its place in
// the interleaved layout.  Walks in the layout's order, which let neighbouring
// waves fill whole lines of scales as in the interleaved quantizer, made
// neighbouring waves read different rows a whole row stride apart: 53.0 us
// (slab-major over all rows) and 55.7 us (slab-major inside groups of 8 rows)
// against 48.7 us row-major for 4096 x 14336 on one box.
template <int LAYOUT>
__global__ __launch_bounds__(kProdThreads) void swiglu_quantize_kernel(
    const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int64_t ld, int rows, int kblocks,
    int nblocks, uint4* __restrict__ y_out, uint32_t* __restrict__ q, uint8_t* __restrict__ scales) {
  constexpr bool PREPACKED = LAYOUT == kLayoutPrepacked;
  const int lane4 = threadIdx.x & 3;
  const int groups_per_grid = gridDim.x * (kProdThreads / 4);
  for (int blk = blockIdx.x * (kProdThreads / 4) + (threadIdx.x >> 2); blk < nblocks;
       blk += kProdUnroll * groups_per_grid) {
    uint4 gv[kProdUnroll], uv[kProdUnroll];
#pragma unroll
    for (int u = 0; u < kProdUnroll; ++u) {
      int b = blk + u * groups_per_grid;
      // out-of-range groups, and the padding rows of a prepacked output, load block 0
      b = (b < nblocks && b / kblocks < rows) ? b : 0;
      const int row = b / kblocks, kb = b - row * kblocks;
      const int64_t off = (int64_t)row * ld + kb * 32 + lane4 * 8;
      // gate and up are read once: non-temporal (same-box A/B on 4096 x 14336: 48.6-49.2 vs 54.4-55.0 us;
      // the same policy on the RMSNorm kernel's loads measured 8 % slower and is not used there)
      const v4i gt = __builtin_nontemporal_load((const v4i*)(gate + off));
      const v4i ut = __builtin_nontemporal_load((const v4i*)(up + off));
      gv[u] = make_uint4((uint32_t)gt.x, (uint32_t)gt.y, (uint32_t)gt.z, (uint32_t)gt.w);
      uv[u] = make_uint4((uint32_t)ut.x, (uint32_t)ut.y, (uint32_t)ut.z, (uint32_t)ut.w);
    }
#pragma unroll
    for (int u = 0; u < kProdUnroll; ++u) {
      const int b = blk + u * groups_per_grid;
      const uint4 y = make_uint4(swiglu_bf16x2(gv[u].x, uv[u].x), swiglu_bf16x2(gv[u].y, uv[u].y),
                                 swiglu_bf16x2(gv[u].z, uv[u].z), swiglu_bf16x2(gv[u].w, uv[u].w));
      uint32_t sbyte;
      uint32_t codes = quantize8(y, sbyte);
      if (b < nblocks) {
        const int row = b / kblocks;
        if (PREPACKED) {
          if (row >= rows) {   // padding row: a zero block
            codes = 0u;
            sbyte = 0u;
          } else if (y_out) {
            y_out[(int64_t)b * 4 + lane4] = y;
          }
          int64_t word, sidx;
          prepacked_index(row, b - row * kblocks, kblocks / 16, word, sidx);
          q[word + lane4] = codes;
          if (lane4 == 0) scales[sidx] = (uint8_t)sbyte;
        } else {
          if (y_out) y_out[(int64_t)b * 4 + lane4] = y;
          q[(int64_t)b * 4 + lane4] = codes;
          if (lane4 == 0) {
            if (LAYOUT == kLayoutInterleaved) {   // rows * kblocks < 2^31
              const uint32_t row = (uint32_t)b / (uint32_t)kblocks, kb = (uint32_t)b - row * (uint32_t)kblocks;
              scales[(kb >> 4) * (uint32_t)rows * 16 + row * 16 + (kb & 15)] = (uint8_t)sbyte;
            } else {
              scales[b] = (uint8_t)sbyte;
            }
          }
        }
      }
    }
  }
}

}  // namespace

template <int SLOTS, int LAYOUT>
void launch_rmsnorm_slots(const void* x, const void* residual, const void* gamma, float eps, int rows, int k,
                          void* h_out, void* y_out, void* q, void* scales, hipStream_t stream) {
  constexpr bool PREPACKED = LAYOUT == kLayoutPrepacked;
  // prepacked: one more workgroup per padding row of the last 64-row panel
  const unsigned grid = PREPACKED ? (unsigned)((rows + 63) / 64 * 64) : (unsigned)rows;
  if (residual)
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<true, SLOTS, LAYOUT>), dim3(grid), dim3(kNormThreads), 0, stream,
                       (const uint4*)x, (const uint4*)residual, (const uint4*)gamma, eps, rows, k, (uint4*)h_out,
                       (uint4*)y_out, (uint32_t*)q, (uint8_t*)scales);
  else
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<false, SLOTS, LAYOUT>), dim3(grid), dim3(kNormThreads), 0, stream,
                       (const uint4*)x, (const uint4*)nullptr, (const uint4*)gamma, eps, rows, k, (uint4*)nullptr,
                       (uint4*)y_out, (uint32_t*)q, (uint8_t*)scales);
}

template <int LAYOUT>
void launch_rmsnorm(const void* x, const void* residual, const void* gamma, float eps, int rows, int k,
                    void* h_out, void* y_out, void* q, void* scales, hipStream_t stream) {
  if (k <= 2 * 8 * kNormThreads)
    launch_rmsnorm_slots<2, LAYOUT>(x, residual, gamma, eps, rows, k, h_out, y_out, q, scales, stream);
  else if (k <= 4 * 8 * kNormThreads)
    launch_rmsnorm_slots<4, LAYOUT>(x, residual, gamma, eps, rows, k, h_out, y_out, q, scales, stream);
  else
    launch_rmsnorm_slots<kNormMaxSlots, LAYOUT>(x, residual, gamma, eps, rows, k, h_out, y_out, q, scales, stream);
}

// Rows stay in registers: 2, 4 or 16 chunks of 8 elements per thread (k up
// to 4096, 8192 or 32768), so the common widths keep the register count, and
// with it the rows in flight per CU, low.
hipError_t launch_rmsnorm_quantize(const void* x, const void* residual, const void* gamma, float eps, int rows, int k,
                                   void* h_out, void* y_out, void* q, void* scales, int layout,
                                   hipStream_t stream) {
  if (!grid_fits((int64_t)(rows + 63) / 64 * 64, kNormThreads)) return hipErrorInvalidConfiguration;
  if (layout != kLayoutRowMajor && k % 512) return hipErrorInvalidValue;
  if (layout == kLayoutInterleaved && (int64_t)rows * (k / 32) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (layout == kLayoutPrepacked)
    launch_rmsnorm<kLayoutPrepacked>(x, residual, gamma, eps, rows, k, h_out, y_out, q, scales, stream);
  else if (layout == kLayoutInterleaved)
    launch_rmsnorm<kLayoutInterleaved>(x, residual, gamma, eps, rows, k, h_out, y_out, q, scales, stream);
  else
    launch_rmsnorm<kLayoutRowMajor>(x, residual, gamma, eps, rows, k, h_out, y_out, q, scales, stream);
  return hipGetLastError();
}

hipError_t launch_swiglu_quantize(const void* gate, const void* up, int64_t ld, int rows, int k, void* y_out, void* q,
                                  void* scales, int layout, hipStream_t stream, int num_cus) {
  const bool prepacked = layout == kLayoutPrepacked;
  if (layout != kLayoutRowMajor && k % 512) return hipErrorInvalidValue;
  const int kblocks = k / 32;
  // the host keeps this at most 2^30 (prepacked: rows rounded up to 64)
  const int nblocks = (prepacked ? (rows + 63) / 64 * 64 : rows) * kblocks;
  const int64_t groups_needed = ((int64_t)nblocks + kProdUnroll - 1) / kProdUnroll;
  int64_t grid = (groups_needed + (kProdThreads / 4) - 1) / (kProdThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  const auto kernel = prepacked ? swiglu_quantize_kernel<kLayoutPrepacked>
                                 : (layout == kLayoutInterleaved ? swiglu_quantize_kernel<kLayoutInterleaved>
                                                                 : swiglu_quantize_kernel<kLayoutRowMajor>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kProdThreads), 0, stream, (const uint16_t*)gate,
                     (const uint16_t*)up, ld, rows, kblocks, nblocks, (uint4*)y_out, (uint32_t*)q, (uint8_t*)scales);
  return hipGetLastError();
}

}  // namespace mxfp4
