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
//  route:    four lanes per token, each keeping the top k of a contiguous
//            quarter of the experts in registers: each logit, mapped to an
//            order-preserving integer key, enters or climbs the descending list
//            only when strictly greater, so equal logits go to the lower id.
//            Two DPP quad merges combine the quarters.  Gate weights are the
//            softmax of the k selected logits in fp32.
//  permute:  one workgroup per expert stages the flat id array in LDS
//            (chunks of 32768, one padded row of 32 consecutive entries per
//            thread of 1024): a count of the kept ids below its expert gives its
//            segment's first row, then one block-wide prefix scan per chunk in
//            (token, slot) order numbers its rows.  Rows of an expert are therefore in ascending token order
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

constexpr int kRouteLanes = 8;       // lanes per token (one half-row)
constexpr int kRouteThreads = 256;   // 32 tokens per workgroup

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

// One candidate into the descending top-K list.  Keys carry the logit's order
// key above a presence bit (an empty slot is 0, below every logit), so the
// first K candidates always fill the list.  A candidate passes an entry only
// when strictly greater: candidates offered in ascending expert id lose ties
// to the entries already held.  Branch-free over the K slots; every
// comparison uses the old list.
template <int K>
__device__ __forceinline__ void topk_insert(uint64_t (&bk)[K], int (&bi)[K], uint64_t c, int e) {
  bool gt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) gt[j] = c > bk[j];
#pragma unroll
  for (int j = K - 1; j >= 0; --j) {
    if (gt[j]) {
      const bool shift = j > 0 && gt[j > 0 ? j - 1 : 0];
      bk[j] = shift ? bk[j > 0 ? j - 1 : 0] : c;
      bi[j] = shift ? bi[j > 0 ? j - 1 : 0] : e;
    }
  }
}

// Merge the partner lane's top-K list (DPP control CTRL) into this one.
// The lane whose bit MASK is clear holds the lower expert ids; both lanes end
// with that lane's list as the base and the other's entries inserted into it
// in order, so ties keep going to the lower id.
template <int K, int CTRL, int MASK>
__device__ __forceinline__ void topk_merge(uint64_t (&bk)[K], int (&bi)[K], int lane) {
  uint64_t ok[K];
  int oi[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)bk[j], CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(bk[j] >> 32), CTRL, 0xF, 0xF, false);
    ok[j] = ((uint64_t)hi << 32) | lo;
    oi[j] = __builtin_amdgcn_mov_dpp(bi[j], CTRL, 0xF, 0xF, false);
  }
  const bool upper = (lane & MASK) != 0;
  uint64_t base_k[K], add_k[K];
  int base_i[K], add_i[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    base_k[j] = upper ? ok[j] : bk[j];
    base_i[j] = upper ? oi[j] : bi[j];
    add_k[j] = upper ? bk[j] : ok[j];
    add_i[j] = upper ? bi[j] : oi[j];
  }
#pragma unroll
  for (int j = 0; j < K; ++j) topk_insert<K>(base_k, base_i, add_k[j], add_i[j]);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    bk[j] = base_k[j];
    bi[j] = base_i[j];
  }
}

// Eight lanes (one half-row) per token: lane L takes the contiguous experts
// [L * span, (L + 1) * span), keeps their top K in registers, then three
// merges (lanes 2i+1 into 2i, then pairs within a quad, then the quads through
// the half-row mirror, lane i with lane 7 - i) give every lane the token's top
// K.  Eight lanes rather than four halve each lane's serial insertions and
// double the waves on the chip.
template <int K, bool VEC>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits, int tokens,
                                                             int experts, int32_t* __restrict__ ids,
                                                             float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRouteThreads / kRouteLanes) + (threadIdx.x / kRouteLanes);
  if (t >= tokens) return;   // uniform over the token's lanes
  const int q = lane & (kRouteLanes - 1);
  const int span = (experts + kRouteLanes - 1) / kRouteLanes;
  const int e_lo = min(q * span, experts), e_hi = min(e_lo + span, experts);
  const float* row = logits + (int64_t)t * experts;
  uint64_t bk[K];
  int bi[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    bk[j] = 0;
    bi[j] = 0;
  }
  if (VEC) {   // experts % 32 == 0 and 16-byte aligned rows: span is a multiple of 4
    for (int e0 = e_lo; e0 < e_hi; e0 += 16) {
      float v[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 f = (e0 + 4 * c < e_hi) ? *(const float4*)(row + e0 + 4 * c) : make_float4(0, 0, 0, 0);
        v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (e0 + u < e_hi) topk_insert<K>(bk, bi, ((uint64_t)order_key(v[u]) << 1) | 1u, e0 + u);
    }
  } else {
    for (int e = e_lo; e < e_hi; ++e) topk_insert<K>(bk, bi, ((uint64_t)order_key(row[e]) << 1) | 1u, e);
  }
  topk_merge<K, 0xB1, 1>(bk, bi, lane);   // quad lanes 1,0,3,2
  topk_merge<K, 0x4E, 2>(bk, bi, lane);   // quad lanes 2,3,0,1
  topk_merge<K, 0x141, 4>(bk, bi, lane);  // half-row mirror: lane i <-> 7 - i, the other quad
  // softmax of the selected logits; the first is the largest
  const float top = key_value((uint32_t)(bk[0] >> 1));
  float ex[K];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    ex[j] = expf(key_value((uint32_t)(bk[j] >> 1)) - top);
    sum += ex[j];
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if ((j & (kRouteLanes - 1)) == q) {
      ids[(int64_t)t * K + j] = bi[j];
      weights[(int64_t)t * K + j] = ex[j] / sum;
    }
  }
}

// ---------------------------------------------------------------------------
// permutation
// ---------------------------------------------------------------------------

constexpr int kPermThreads = 1024;                   // 16 waves: 4 per SIMD hide the LDS and memory latency
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermSeg = 32;                         // consecutive entries per thread per chunk
constexpr int kPermChunk = kPermThreads * kPermSeg;  // entries per chunk (32768)
constexpr int kPermPitch = kPermSeg + 1;             // LDS words per thread segment (odd: no bank conflicts)
constexpr int kPermLds = kPermThreads * kPermPitch * 4;

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
  int total = 0;
#pragma unroll
  for (int q = 0; q < kPermWaves; ++q) total += red[q];
  __syncthreads();
  return total;
}

// Ids [c0, c0 + 32768) into LDS, entry c0 + i at word (i / 32) * 33 + i % 32,
// so thread t's 32 consecutive entries form one padded row; entries past n
// read as -1 (dropped).  Coalesced 16-byte loads, eight in flight per thread.
template <bool VEC>
__device__ __forceinline__ void stage_chunk(const int32_t* __restrict__ ids, int n, int c0, int* lds) {
  __syncthreads();   // the previous chunk is no longer read
  for (int q0 = 0; q0 < kPermChunk / 4; q0 += 8 * kPermThreads) {
    int4 x[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int i = c0 + 4 * (q0 + a * kPermThreads + threadIdx.x);
      if (VEC && i + 4 <= n) {
        x[a] = *(const int4*)(ids + i);
      } else {
        x[a].x = (i < n) ? ids[i] : -1;
        x[a].y = (i + 1 < n) ? ids[i + 1] : -1;
        x[a].z = (i + 2 < n) ? ids[i + 2] : -1;
        x[a].w = (i + 3 < n) ? ids[i + 3] : -1;
      }
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int l = 4 * (q0 + a * kPermThreads + threadIdx.x);   // 4 entries, all in one thread row
      int* dst = lds + (l / kPermSeg) * kPermPitch + (l % kPermSeg);
      dst[0] = x[a].x; dst[1] = x[a].y; dst[2] = x[a].z; dst[3] = x[a].w;
    }
  }
  __syncthreads();
}

// Workgroup e < experts numbers the rows of expert e; workgroup `experts`
// writes the segment end, marks dropped entries and clears unused row slots.
// The ids go through LDS in chunks of 32768; when all of them fit one chunk
// they are staged once and serve both passes.
template <bool VEC>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int n, int top_k,
                                                              int experts, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ token_rows) {
  extern __shared__ __attribute__((aligned(16))) int lds_ids[];
  __shared__ int red[kPermWaves];
  __shared__ int wave_tot[2][kPermWaves];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool one_chunk = n <= kPermChunk;
  const int* mine_row = lds_ids + tid * kPermPitch;

  // kept ids below e: the first row of expert e (for e == experts, every kept id)
  int cnt = 0;
  for (int c0 = 0; c0 < n; c0 += kPermChunk) {
    stage_chunk<VEC>(ids, n, c0, lds_ids);
#pragma unroll 8
    for (int u = 0; u < kPermSeg; ++u) {
      const int v = mine_row[u];
      cnt += (v >= 0 && v < e) ? 1 : 0;
    }
  }
  const int base = block_sum(cnt, red);
  if (tid == 0) offsets[e] = base;

  if (e == experts) {
    for (int i = base + tid; i < n; i += kPermThreads) row_token[i] = -1;
    for (int c0 = 0; c0 < n; c0 += kPermChunk) {
      if (!one_chunk) stage_chunk<VEC>(ids, n, c0, lds_ids);
      const int i0 = c0 + tid * kPermSeg;
#pragma unroll 8
      for (int u = 0; u < kPermSeg; ++u) {
        const int v = mine_row[u];
        if ((v < 0 || v >= experts) && i0 + u < n) token_rows[i0 + u] = -1;
      }
    }
    return;
  }

  // number the entries of expert e in flat (token, slot) order: one block-wide
  // exclusive scan of per-thread match counts per chunk
  int run = base;
  int parity = 0;
  for (int c0 = 0; c0 < n; c0 += kPermChunk, parity ^= 1) {
    if (!one_chunk) stage_chunk<VEC>(ids, n, c0, lds_ids);
    int mine = 0;
#pragma unroll 8
    for (int u = 0; u < kPermSeg; ++u) mine += (mine_row[u] == e) ? 1 : 0;
    const int incl = wave_incl_scan(mine, lane);
    if (lane == 63) wave_tot[parity][w] = incl;
    __syncthreads();   // the other parity's totals are not rewritten before the next barrier
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < kPermWaves; ++q) {
      const int tq = wave_tot[parity][q];
      before += (q < w) ? tq : 0;
      total += tq;
    }
    if (mine > 0) {
      int r = run + before + incl - mine;
      const int i0 = c0 + tid * kPermSeg;
      for (int u = 0; u < kPermSeg; ++u) {
        if (mine_row[u] == e) {
          row_token[r] = (i0 + u) / top_k;
          token_rows[i0 + u] = r;
          ++r;
        }
      }
    }
    run += total;
  }
}

// ---------------------------------------------------------------------------
// quantization scattered into the expert-sorted rows
// ---------------------------------------------------------------------------

constexpr int kScatterThreads = 256;
constexpr int kScatterUnroll = 4;
constexpr int kScatterSlots = 4;   // slots whose destination rows are loaded with the blocks

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
// biased exponent E.  IL: scale bytes in the interleaved layout
// [k/512, total_rows, 16].
template <bool FP8, bool IL>
__global__ __launch_bounds__(kScatterThreads) void quantize_scatter_kernel(
    const uint4* __restrict__ x, int kblocks, int nblocks, int top_k, const int32_t* __restrict__ token_rows,
    int total_rows, uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  const int lane4 = threadIdx.x & 3;
  const int groups_per_grid = gridDim.x * (kScatterThreads / 4);
  // kScatterUnroll blocks per lane group per iteration: all their loads are in
  // flight before any block's stores (4 measured 7 % faster than 2)
  for (int blk = blockIdx.x * (kScatterThreads / 4) + (threadIdx.x >> 2); blk < nblocks;
       blk += kScatterUnroll * groups_per_grid) {
    uint4 v[kScatterUnroll];
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      const int b = blk + u * groups_per_grid;
      v[u] = x[(int64_t)(b < nblocks ? b : 0) * 4 + lane4];   // out-of-range groups load block 0, store nothing
    }
    // the destination rows of the first kScatterSlots slots of every block,
    // loaded with the blocks rather than one slot at a time before each store
    int rws[kScatterUnroll][kScatterSlots];
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      const int b = blk + u * groups_per_grid;
      const int t = b / kblocks;
#pragma unroll
      for (int j = 0; j < kScatterSlots; ++j)
        rws[u][j] = (b < nblocks && j < top_k) ? token_rows[(int64_t)t * top_k + j] : -1;
    }
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      const int b = blk + u * groups_per_grid;
      const int t = b / kblocks, kb = b - t * kblocks;
      const uint32_t m = umax16x2(umax16x2(v[u].x & 0x7FFF7FFFu, v[u].y & 0x7FFF7FFFu),
                                  umax16x2(v[u].z & 0x7FFF7FFFu, v[u].w & 0x7FFF7FFFu));
      const uint32_t amax_bits = quad_max(max(m & 0xFFFFu, m >> 16));
      const int exp_field = (int)(amax_bits >> 7);
      const uint32_t sbyte = (uint32_t)max(exp_field - (FP8 ? 8 : 2), 0);
      const float scale = __uint_as_float(sbyte << 23);
      uint2 codes8 = make_uint2(0u, 0u);
      uint32_t codes4 = 0;
      if constexpr (FP8) {
        const uint32_t bound = ((8u + sbyte) << 7) | 0x60u;   // 448 * 2^e as BF16 magnitude bits
        codes8.x = cvt_fp8x4(clamp_mag16x2(v[u].x, bound), clamp_mag16x2(v[u].y, bound), scale);
        codes8.y = cvt_fp8x4(clamp_mag16x2(v[u].z, bound), clamp_mag16x2(v[u].w, bound), scale);
      } else {
        codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v[u].x), scale, 0);
        codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v[u].y), scale, 1);
        codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v[u].z), scale, 2);
        codes4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(codes4, __builtin_bit_cast(bf16x2_t, v[u].w), scale, 3);
      }
      if (b >= nblocks) continue;   // uniform over the lane group
      for (int j = 0; j < top_k; ++j) {
        int r;
        if (j < kScatterSlots) {
          r = -1;
#pragma unroll
          for (int i = 0; i < kScatterSlots; ++i) r = (i == j) ? rws[u][i] : r;
        } else {
          r = token_rows[(int64_t)t * top_k + j];
        }
        if (r < 0 || r >= total_rows) continue;   // dropped entry (or a malformed row index)
        if constexpr (FP8) {
          *(uint2*)(q + (int64_t)r * kblocks * 32 + kb * 32 + lane4 * 8) = codes8;
        } else {
          *(uint32_t*)(q + (int64_t)r * kblocks * 16 + kb * 16 + lane4 * 4) = codes4;
        }
        if (lane4 == 0) {
          if constexpr (IL)   // interleaved [k/512, total_rows, 16]: total_rows * k/32 < 2^31
            scales[(uint32_t)(kb >> 4) * (uint32_t)total_rows * 16 + (uint32_t)r * 16 + (kb & 15)] = (uint8_t)sbyte;
          else
            scales[(int64_t)r * kblocks + kb] = (uint8_t)sbyte;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------

constexpr int kCombineThreads = 256;
constexpr int kCombineSlots = 8;   // slots whose rows are loaded together

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
  // per group of kCombineSlots slots, all row indices and then all row loads
  // are issued before the group's first sum: up to kCombineSlots independent
  // 16-byte loads in flight per lane instead of one index-then-row chain per
  // slot.  The sums still run in slot order.
  for (int j0 = 0; j0 < top_k; j0 += kCombineSlots) {
    int rows[kCombineSlots];
    float wts[kCombineSlots];
#pragma unroll
    for (int j = 0; j < kCombineSlots; ++j) {
      rows[j] = -1;
      wts[j] = 0.0f;
      if (j0 + j < top_k) {
        const int64_t slot = (int64_t)t * top_k + j0 + j;
        const int r = token_rows[slot];
        rows[j] = (r >= 0 && r < total_rows) ? r : -1;
        wts[j] = weights[slot];
      }
    }
    uint32_t word[kCombineSlots][4];
#pragma unroll
    for (int j = 0; j < kCombineSlots; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) word[j][e] = 0u;
      if (rows[j] < 0) continue;
      const uint16_t* src = y + (int64_t)rows[j] * n + col0;
      if (VEC) {
        // each expert-output row is read once: non-temporal (same-box A/B on
        // the MoE workload's combine: 45.4-47.3 vs 48.6-50.0 us)
        const v4i v = __builtin_nontemporal_load((const v4i*)src);
        word[j][0] = (uint32_t)v.x; word[j][1] = (uint32_t)v.y; word[j][2] = (uint32_t)v.z; word[j][3] = (uint32_t)v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (2 * e < cnt) ? src[2 * e] : 0u;
          const uint32_t hi = (2 * e + 1 < cnt) ? src[2 * e + 1] : 0u;
          word[j][e] = lo | (hi << 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kCombineSlots; ++j) {
      if (rows[j] < 0) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yv = __uint_as_float(((word[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
        acc[e] = fmaf(wts[j], yv, acc[e]);
      }
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

template <int K>
hipError_t launch_route_k(const float* logits, int tokens, int experts, int32_t* ids, float* weights,
                          hipStream_t stream) {
  const int64_t blocks = ((int64_t)tokens + kRouteThreads / kRouteLanes - 1) / (kRouteThreads / kRouteLanes);
  if (!grid_fits(blocks, kRouteThreads)) return hipErrorInvalidConfiguration;
  const bool vec = experts % (4 * kRouteLanes) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((route_kernel<K, true>), dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream, logits,
                       tokens, experts, ids, weights);
  else
    hipLaunchKernelGGL((route_kernel<K, false>), dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream, logits,
                       tokens, experts, ids, weights);
  return hipGetLastError();
}

hipError_t launch_moe_route(const float* logits, int tokens, int experts, int top_k, int32_t* ids, float* weights,
                            hipStream_t stream) {
  switch (top_k) {
    case 1: return launch_route_k<1>(logits, tokens, experts, ids, weights, stream);
    case 2: return launch_route_k<2>(logits, tokens, experts, ids, weights, stream);
    case 3: return launch_route_k<3>(logits, tokens, experts, ids, weights, stream);
    case 4: return launch_route_k<4>(logits, tokens, experts, ids, weights, stream);
    case 5: return launch_route_k<5>(logits, tokens, experts, ids, weights, stream);
    case 6: return launch_route_k<6>(logits, tokens, experts, ids, weights, stream);
    case 7: return launch_route_k<7>(logits, tokens, experts, ids, weights, stream);
    case 8: return launch_route_k<8>(logits, tokens, experts, ids, weights, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_moe_permute(const int32_t* ids, int n, int top_k, int experts, int32_t* offsets,
                              int32_t* row_token, int32_t* token_rows, hipStream_t stream) {
  const bool vec = (reinterpret_cast<uintptr_t>(ids) & 15) == 0;
  const auto kernel = vec ? permute_kernel<true> : permute_kernel<false>;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kPermLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(experts + 1)), dim3(kPermThreads), kPermLds, stream, ids, n, top_k,
                     experts, offsets, row_token, token_rows);
  return hipGetLastError();
}

hipError_t launch_moe_quantize_scatter(const void* x, int tokens, int k, int top_k, const int32_t* token_rows,
                                       int total_rows, void* q, void* scales, bool fp8, hipStream_t stream,
                                       int num_cus, bool interleaved) {
  const int kblocks = k / 32;
  if (interleaved && (k % 512 != 0 || (int64_t)total_rows * kblocks >= ((int64_t)1 << 31)))
    return hipErrorInvalidValue;
  const int nblocks = tokens * kblocks;   // the host keeps this below 2^31
  const int64_t groups_needed = ((int64_t)nblocks + kScatterUnroll - 1) / kScatterUnroll;
  int64_t grid = (groups_needed + (kScatterThreads / 4) - 1) / (kScatterThreads / 4);
  const int64_t max_grid = (int64_t)num_cus * 8;
  if (grid > max_grid) grid = max_grid;
  if (grid < 1) grid = 1;
  const auto kernel = fp8 ? (interleaved ? quantize_scatter_kernel<true, true> : quantize_scatter_kernel<true, false>)
                          : (interleaved ? quantize_scatter_kernel<false, true> : quantize_scatter_kernel<false, false>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kScatterThreads), 0, stream, (const uint4*)x, kblocks,
                     nblocks, top_k, token_rows, total_rows, (uint8_t*)q, (uint8_t*)scales);
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
