// MoE steps around the grouped block-scaled GEMM (gfx950): top-k routing,
// the expert-sorted row permutation, quantization scattered straight into the
// grouped GEMM's operand rows, and the weighted combine of expert outputs.
//
// The grouped GEMM takes the rows of every expert as one contiguous segment
// (quadbit README, "Distributed sparse-FP4 MoE": a segmented routed-row
// kernel, one launch), and its activation operand is the per-expert
// quantized tile ("fp4_quantization" Mojo module page,
// grouped_quantize_dynamic_scaled_fp4_async).  The steps here produce that
// layout on the device and fold the expert outputs back per token:
//
//  route:    one wave per token; lane e holds logits e, e + 64, e + 128,
//            e + 192.  Each of the k rounds takes a wave-wide max of a 64-bit
//            key (order-preserving integer image of the logit, then 0xFFFF - id
//            so equal logits go to the lower id) and removes the winner.  Gate
//            weights are the softmax of the k selected logits in fp32.
//  permute:  one workgroup per expert scans the flat id array twice: a count
//            of the kept ids below its expert (its segment's first row), then
//            a block-wide prefix scan in (token, slot) order that numbers its
//            rows.  Rows of an expert are therefore in ascending token order
//            and the result does not depend on timing.  One extra workgroup
//            writes the segment end, marks dropped entries and clears the
//            unused row slots.
//  quantize: the quantizer's mapping (4 lanes per 32-element block, amax by
//            integer max, the CDNA4 scaled converts) over the token rows, each
//            block quantized once and stored to every row its token was routed
//            to: the activations are read once instead of once per route.
//  combine:  one lane per 8 output columns of a token; fp32 fused
//            multiply-adds over the token's slots in slot order, BF16 (nearest
//            even) or fp32 out.  All four are bandwidth-bound.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

// ---------------------------------------------------------------------------
// routing
// ---------------------------------------------------------------------------

constexpr int kRouteThreads = 256;   // 4 tokens per workgroup, one wave each

// Order-preserving map of a float onto uint32 (negative zero taken as +0, so
// the two zeros tie as they compare equal).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off);
    v = umax64(v, ((uint64_t)hi << 32) | lo);
  }
  return v;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits, int tokens,
                                                             int experts, int top_k, int32_t* __restrict__ ids,
                                                             float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  if (t >= tokens) return;   // wave-uniform
  const float* row = logits + (int64_t)t * experts;
  // key 0 = no candidate; every real candidate is at least 0xFFFF - 255
  uint64_t cand[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    cand[i] = (e < experts) ? (((uint64_t)order_key(row[e]) << 16) | (uint64_t)(0xFFFF - e)) : 0;
  }
  int sel_id[kMoeMaxTopK];
  float sel_val[kMoeMaxTopK];
#pragma unroll
  for (int j = 0; j < kMoeMaxTopK; ++j) {
    sel_id[j] = 0;
    sel_val[j] = 0.0f;
    if (j < top_k) {
      const uint64_t best = wave_max_u64(umax64(umax64(cand[0], cand[1]), umax64(cand[2], cand[3])));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (cand[i] == best) cand[i] = 0;   // ids are distinct, so only the winner matches
      sel_id[j] = 0xFFFF - (int)(best & 0xFFFFu);
      sel_val[j] = key_value((uint32_t)(best >> 16));
    }
  }
  // softmax of the selected logits; the first is the largest
  float ex[kMoeMaxTopK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMoeMaxTopK; ++j) {
    ex[j] = (j < top_k) ? expf(sel_val[j] - sel_val[0]) : 0.0f;
    sum += ex[j];
  }
#pragma unroll
  for (int j = 0; j < kMoeMaxTopK; ++j) {
    if (j < top_k && lane == j) {
      ids[(int64_t)t * top_k + j] = sel_id[j];
      weights[(int64_t)t * top_k + j] = ex[j] / sum;
    }
  }
}

// ---------------------------------------------------------------------------
// permutation
// ---------------------------------------------------------------------------

constexpr int kPermThreads = 256;
constexpr int kPermPerThread = 4;

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const int total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int n, int top_k,
                                                              int experts, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ token_rows) {
  __shared__ int red[4];
  __shared__ int wave_tot[2][4];
  const int e = blockIdx.x;   // e == experts: segment end, dropped entries, unused rows
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // kept ids below e: the first row of expert e (for e == experts, all kept ids)
  int cnt = 0;
  for (int i = tid; i < n; i += kPermThreads) {
    const int v = ids[i];
    cnt += (v >= 0 && v < e) ? 1 : 0;
  }
  const int base = block_sum(cnt, red);
  if (tid == 0) offsets[e] = base;

  if (e == experts) {
    for (int i = base + tid; i < n; i += kPermThreads) row_token[i] = -1;
    for (int i = tid; i < n; i += kPermThreads) {
      const int v = ids[i];
      if (v < 0 || v >= experts) token_rows[i] = -1;
    }
    return;
  }

  // number the entries of expert e in flat (token, slot) order
  int run = base;
  int parity = 0;
  for (int c0 = 0; c0 < n; c0 += kPermThreads * kPermPerThread, parity ^= 1) {
    int v[kPermPerThread];
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kPermPerThread; ++u) {
      const int i = c0 + tid * kPermPerThread + u;
      v[u] = (i < n) ? ids[i] : -1;
      mine += (v[u] == e) ? 1 : 0;
    }
    const int incl = wave_incl_scan(mine, lane);
    if (lane == 63) wave_tot[parity][w] = incl;
    __syncthreads();   // the other parity's totals are not rewritten before the next barrier
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tq = wave_tot[parity][q];
      before += (q < w) ? tq : 0;
      total += tq;
    }
    int r = run + before + incl - mine;
#pragma unroll
    for (int u = 0; u < kPermPerThread; ++u) {
      if (v[u] == e) {
        const int i = c0 + tid * kPermPerThread + u;
        row_token[r] = i / top_k;
        token_rows[i] = r;
        ++r;
      }
    }
    run += total;
  }
}

// ---------------------------------------------------------------------------
// quantization scattered into the expert-sorted rows
// ---------------------------------------------------------------------------

constexpr int kScatterThreads = 256;

__device__ __forceinline__ uint32_t umax16x2(uint32_t a, uint32_t b) {
  return max(a & 0xFFFFu, b & 0xFFFFu) | (max(a >> 16, b >> 16) << 16);
}

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // lane ^ 1
  v = max(v, o);
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);            // lane ^ 2
  return max(v, o);
}

__device__ __forceinline__ uint32_t clamp_mag16x2(uint32_t w, uint32_t bound) {
  const uint32_t lo = min(w & 0x7FFFu, bound) | (w & 0x8000u);
  const uint32_t hi = min((w >> 16) & 0x7FFFu, bound) | ((w >> 16) & 0x8000u);
  return lo | (hi << 16);
}

typedef short short2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_fp8x4(uint32_t w01, uint32_t w23, float scale) {
  short2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w01), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w23), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// FP8 = false: MXFP4 rows (K/2 code bytes, 4 per lane); true: MXFP8 rows
// (K code bytes, 8 per lane).  Scale rule and converts as in the dense
// quantizers: byte = max(E - 2, 0) (FP4) or max(E - 8, 0) (FP8) for amax's
// biased exponent E.
template <bool FP8>
__global__ __launch_bounds__(kScatterThreads) void quantize_scatter_kernel(
    const uint4* __restrict__ x, int kblocks, int nblocks, int top_k, const int32_t* __restrict__ token_rows,
    int total_rows, uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  const int lane4 = threadIdx.x & 3;
  const int groups_per_grid = gridDim.x * (kScatterThreads / 4);
  for (int b = blockIdx.x * (kScatterThreads / 4) + (threadIdx.x >> 2); b < nblocks; b += groups_per_grid) {
    const uint4 v = x[(int64_t)b * 4 + lane4];
    const int t = b / kblocks, kb = b - t * kblocks;
    const uint32_t m = umax16x2(umax16x2(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                umax16x2(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
    const uint32_t amax_bits = quad_max(max(m & 0xFFFFu, m >> 16));
    const int exp_field = (int)(amax_bits >> 7);
    const uint32_t sbyte = (uint32_t)max(exp_field - (FP8 ? 8 : 2), 0);
    const float scale = __uint_as_float(sbyte << 23);
    uint2 codes8 = make_uint2(0u, 0u);
    uint32_t codes4 = 0;
    if constexpr (FP8) {
      const uint32_t bound = ((8u + sbyte) << 7) | 0x60u;   // 448 * 2^e as BF16 magnitude bits
      codes8.x = cvt_fp8x4(clamp_mag16x2(v.x, bound), clamp_mag16x2(v.y, bound), scale);
      codes8.y = cvt_fp8x4(clamp_mag16x2(v.z, bound), clamp_mag16x2(v.w, bound), scale);
    } else {
      codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v.x), scale, 0);
      codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v.y), scale, 1);
      codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v.z), scale, 2);
      codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v.w), scale, 3);
    }
    for (int j = 0; j < top_k; ++j) {
      const int r = token_rows[(int64_t)t * top_k + j];
      if (r < 0 || r >= total_rows) continue;   // dropped entry (or a malformed row index)
      if constexpr (FP8) {
        *(uint2*)(q + (int64_t)r * kblocks * 32 + kb * 32 + lane4 * 8) = codes8;
      } else {
        *(uint32_t*)(q + (int64_t)r * kblocks * 16 + kb * 16 + lane4 * 4) = codes4;
      }
      if (lane4 == 0) scales[(int64_t)r * kblocks + kb] = (uint8_t)sbyte;
    }
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------

constexpr int kCombineThreads = 256;

template <bool F32_OUT, bool VEC>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y, int total_rows,
                                                                 int n, const int32_t* __restrict__ token_rows,
                                                                 const float* __restrict__ weights, int tokens,
                                                                 int top_k, void* __restrict__ out) {
  const int chunks = (n + 7) >> 3;
  const int idx = blockIdx.x * kCombineThreads + threadIdx.x;
  if (idx >= tokens * chunks) return;
  const int t = idx / chunks, c = idx - t * chunks;
  const int col0 = c * 8;
  const int cnt = min(8, n - col0);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    const int r = token_rows[(int64_t)t * top_k + j];
    if (r < 0 || r >= total_rows) continue;
    const float w = weights[(int64_t)t * top_k + j];
    const uint16_t* src = y + (int64_t)r * n + col0;
    uint32_t word[4];
    if (VEC) {
      const uint4 v = *(const uint4*)src;
      word[0] = v.x; word[1] = v.y; word[2] = v.z; word[3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (2 * e < cnt) ? src[2 * e] : 0u;
        const uint32_t hi = (2 * e + 1 < cnt) ? src[2 * e + 1] : 0u;
        word[e] = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float yv = __uint_as_float(((word[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
      acc[e] = fmaf(w, yv, acc[e]);
    }
  }
  if (F32_OUT) {
    float* dst = (float*)out + (int64_t)t * n + col0;
    if (VEC) {
      *(float4*)dst = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *(float4*)(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      for (int e = 0; e < cnt; ++e) dst[e] = acc[e];
    }
  } else {
    uint16_t* dst = (uint16_t*)out + (int64_t)t * n + col0;
    if (VEC) {
      *(uint4*)dst = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      for (int e = 0; e < cnt; ++e) dst[e] = (uint16_t)f32_to_bf16_bits(acc[e]);
    }
  }
}

}  // namespace

hipError_t launch_moe_route(const float* logits, int tokens, int experts, int top_k, int32_t* ids, float* weights,
                            hipStream_t stream) {
  const int64_t blocks = ((int64_t)tokens + 3) / 4;
  if (!grid_fits(blocks, kRouteThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream, logits, tokens, experts,
                     top_k, ids, weights);
  return hipGetLastError();
}

hipError_t launch_moe_permute(const int32_t* ids, int n, int top_k, int experts, int32_t* offsets,
                              int32_t* row_token, int32_t* token_rows, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)(experts + 1)), dim3(kPermThreads), 0, stream, ids, n, top_k,
                     experts, offsets, row_token, token_rows);
  return hipGetLastError();
}

hipError_t launch_moe_quantize_scatter(const void* x, int tokens, int k, int top_k, const int32_t* token_rows,
                                       int total_rows, void* q, void* scales, bool fp8, hipStream_t stream,
                                       int num_cus) {
  const int kblocks = k / 32;
  const int nblocks = tokens * kblocks;   // the host keeps this below 2^31
  int64_t grid = ((int64_t)nblocks + (kScatterThreads / 4) - 1) / (kScatterThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  if (fp8)
    hipLaunchKernelGGL(quantize_scatter_kernel<true>, dim3((unsigned)grid), dim3(kScatterThreads), 0, stream,
                       (const uint4*)x, kblocks, nblocks, top_k, token_rows, total_rows, (uint8_t*)q,
                       (uint8_t*)scales);
  else
    hipLaunchKernelGGL(quantize_scatter_kernel<false>, dim3((unsigned)grid), dim3(kScatterThreads), 0, stream,
                       (const uint4*)x, kblocks, nblocks, top_k, token_rows, total_rows, (uint8_t*)q,
                       (uint8_t*)scales);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* y, int total_rows, int n, const int32_t* token_rows, const float* weights,
                              int tokens, int top_k, void* out, bool f32_out, bool vec, hipStream_t stream) {
  const int64_t threads = (int64_t)tokens * ((n + 7) / 8);   // the host keeps this below 2^31
  const int64_t blocks = (threads + kCombineThreads - 1) / kCombineThreads;
  if (!grid_fits(blocks, kCombineThreads)) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)blocks), b(kCombineThreads);
  const uint16_t* yy = (const uint16_t*)y;
  if (f32_out) {
    if (vec) hipLaunchKernelGGL((combine_kernel<true, true>), g, b, 0, stream, yy, total_rows, n, token_rows, weights, tokens, top_k, out);
    else hipLaunchKernelGGL((combine_kernel<true, false>), g, b, 0, stream, yy, total_rows, n, token_rows, weights, tokens, top_k, out);
  } else {
    if (vec) hipLaunchKernelGGL((combine_kernel<false, true>), g, b, 0, stream, yy, total_rows, n, token_rows, weights, tokens, top_k, out);
    else hipLaunchKernelGGL((combine_kernel<false, false>), g, b, 0, stream, yy, total_rows, n, token_rows, weights, tokens, top_k, out);
  }
  return hipGetLastError();
}

}  // namespace mxfp4
