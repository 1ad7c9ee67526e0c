// LDS-staged block-scaled FP4 GEMM on the CDNA4 scaled MFMA (gfx950).
//
// Computes C[m][n] = sum_k A[m][k] * B[n][k] where both operands are MXFP4:
// packed E2M1 codes plus one E8M0 scale per 32 elements along K ("Packed MXFP4
// & NVFP4 GEMM + mega-MoE" page, Summary: mxfp4_gemm_nt, [M,K] @ [N,K].T, BF16
// out, UE8M0 scales at granularity 32; "fp4_quantization" page,
// matmul_dynamic_block_scaled_mxfp4 and grouped_matmul_block_scaled_mxfp4: the
// dense and per-expert block-scaled matmuls on CDNA4).
//
// Hardware mapping
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4: lane l holds
//    16 bytes (one 32-element K-block) of row l % 32, K-block l / 32, and the
//    E8M0 byte of exactly that (row, block) in its scale register (byte chosen
//    by op_sel).  So a block scale is applied inside the MFMA: no dequantized
//    operand ever exists, and the packed bytes go HBM -> LDS -> VGPR unchanged.
//  * The MFMA's first operand is fed from B and its second from A, so the
//    result lands transposed: lane l holds output row (l % 32) and four runs of
//    four consecutive output columns, which become 8-byte BF16 stores.
//  * A stage covers 128 K elements: 64 code bytes per row and one 32-bit word
//    of four scale bytes per row (one word per 128 K, read as the row's four
//    scale bytes in little-endian order).  Stages are copied global -> LDS with
//    global_load_lds_dwordx4 / _dword, without passing through VGPRs, double
//    buffered so the next stage streams in while the MFMAs consume this one.
//  * LDS rows are 64 bytes = four 16-byte chunks; chunk c of row r is stored
//    at chunk position c ^ swz(r) so the ds_read_b128 of 8 or 16 consecutive
//    rows at one logical chunk touches distinct banks.
//  * 256 threads = 4 waves in a 2x2 grid; each wave owns a (BM/2) x (BN/2)
//    sub-tile as (BM/64) x (BN/64) MFMA blocks of 32x32.
//  * Workgroup -> tile mapping is XCD-aware (see tile_coords in common.hpp).
//
// Ragged edges: rows past M (or N) read a clamped, valid row and are never
// stored.  K must be a multiple of 32; when it is not a multiple of 128 every
// stage goes through a register path that zero-fills the missing 32-blocks
// (zero codes contribute nothing whatever their scale).
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kBK = 128;            // K elements per stage
constexpr int kRowBytes = kBK / 2;  // code bytes per row per stage
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

template <int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int S_BYTES = (BM + BN) * 4;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int A_LOADS = BM * 4 / 64 / 4;       // 16-byte chunk loads per wave per stage
  static constexpr int B_LOADS = BN * 4 / 64 / 4;
  static constexpr int S_LOADS = (BM + BN) / 64 / 4;    // 4-byte scale-word loads per wave per stage
  static constexpr int LOADS = A_LOADS + B_LOADS + S_LOADS;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes");
  static_assert((BM + BN) % 256 == 0, "scale loads must split evenly over 4 waves");
};

// Row range of the A tile a workgroup works on (dense: [m0, min(m0+BM, M));
// grouped: the expert's rows inside this m-tile).
struct RowRange {
  int lo;     // first row of the tile
  int last;   // last valid row (reads are clamped to it)
  int end;    // one past the last row that is stored
};

template <class C>
struct Pointers {
  const uint8_t* a_code[C::A_LOADS];
  const uint8_t* b_code[C::B_LOADS];
  const uint8_t* scale[C::S_LOADS];
};

// Per-lane global source addresses of the DMA copies, for stage 0.
template <class C>
__device__ __forceinline__ void make_pointers(Pointers<C>& p, const uint8_t* a_q, const uint8_t* a_s,
                                              const uint8_t* b_q, const uint8_t* b_s,
                                              const RowRange& ar, int n0, int n, int k) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t kb = k / 2, ks = k / 32;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    const int r = slot >> 2, lc = (slot & 3) ^ swz(r);
    const int row = min(ar.lo + r, ar.last);
    p.a_code[j] = a_q + row * kb + lc * 16;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    const int r = slot >> 2, lc = (slot & 3) ^ swz(r);
    const int row = min(n0 + r, n - 1);
    p.b_code[j] = b_q + row * kb + lc * 16;
  }
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    if (slot < C::BM) {
      const int row = min(ar.lo + slot, ar.last);
      p.scale[j] = a_s + row * ks;
    } else {
      const int row = min(n0 + slot - C::BM, n - 1);
      p.scale[j] = b_s + row * ks;
    }
  }
}

// Stage kt via direct global -> LDS copies (requires k % 128 == 0).
template <class C>
__device__ __forceinline__ void load_stage_dma(uint8_t MXFP4_LDS* stage, const Pointers<C>& p, int kt) {
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j)
    g2lds_16(p.a_code[j] + kt * kRowBytes, (MXFP4_LDS void*)(stage + (j * 4 + w) * 64 * 16));
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j)
    g2lds_16(p.b_code[j] + kt * kRowBytes, (MXFP4_LDS void*)(stage + C::A_BYTES + (j * 4 + w) * 64 * 16));
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j)
    g2lds_4(p.scale[j] + kt * 4, (MXFP4_LDS void*)(stage + C::A_BYTES + C::B_BYTES + (j * 4 + w) * 64 * 4));
}

// Stage kt through registers, any k % 32 == 0: 32-blocks at or past k get zero
// codes and scale byte 127.
template <class C>
__device__ __forceinline__ void load_stage_generic(uint8_t MXFP4_LDS* stage, const Pointers<C>& p,
                                                   int kt, int k) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kblocks_left = k / 32 - kt * 4;    // valid 32-blocks in this stage (may exceed 4)
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    const int lc = (slot & 3) ^ swz(slot >> 2);
    v4i v = {0, 0, 0, 0};
    if (lc < kblocks_left) v = *(const v4i*)(p.a_code[j] + kt * kRowBytes);
    *(v4i MXFP4_LDS*)(stage + slot * 16) = v;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    const int lc = (slot & 3) ^ swz(slot >> 2);
    v4i v = {0, 0, 0, 0};
    if (lc < kblocks_left) v = *(const v4i*)(p.b_code[j] + kt * kRowBytes);
    *(v4i MXFP4_LDS*)(stage + C::A_BYTES + slot * 16) = v;
  }
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = b < kblocks_left ? (uint32_t)p.scale[j][kt * 4 + b] : 127u;
      word |= byte << (8 * b);
    }
    *(uint32_t MXFP4_LDS*)(stage + C::A_BYTES + C::B_BYTES + slot * 4) = word;
  }
}

template <class C, int S>
__device__ __forceinline__ void compute_kstep(const uint8_t MXFP4_LDS* stage, v16f (&acc)[C::MI][C::NI],
                                              const int (&asc)[C::MI], const int (&bsc)[C::NI],
                                              int wm0, int wn0, int lane) {
  const int c = 2 * S + (lane >> 5);
  v4i af[C::MI], bf[C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int r = wm0 + 32 * i + (lane & 31);
    af[i] = *(const v4i MXFP4_LDS*)(stage + r * kRowBytes + ((c ^ swz(r)) << 4));
  }
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int r = wn0 + 32 * j + (lane & 31);
    bf[j] = *(const v4i MXFP4_LDS*)(stage + C::A_BYTES + r * kRowBytes + ((c ^ swz(r)) << 4));
  }
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
      acc[i][j] = mfma32_fp4<2 * S>(bf[j], af[i], acc[i][j], bsc[j], asc[i]);
}

template <class C>
__device__ __forceinline__ void compute_stage(const uint8_t MXFP4_LDS* stage, v16f (&acc)[C::MI][C::NI],
                                              int wm0, int wn0, int lane) {
  const uint32_t MXFP4_LDS* sw = (const uint32_t MXFP4_LDS*)(stage + C::A_BYTES + C::B_BYTES);
  const int shift = 8 * (lane >> 5);   // lanes 32..63 hold the odd 32-blocks
  int asc[C::MI], bsc[C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) asc[i] = (int)(sw[wm0 + 32 * i + (lane & 31)] >> shift);
#pragma unroll
  for (int j = 0; j < C::NI; ++j) bsc[j] = (int)(sw[C::BM + wn0 + 32 * j + (lane & 31)] >> shift);
  compute_kstep<C, 0>(stage, acc, asc, bsc, wm0, wn0, lane);
  compute_kstep<C, 1>(stage, acc, asc, bsc, wm0, wn0, lane);
}

template <class C>
__device__ __forceinline__ void store_tile(const GemmArgs& args, const v16f (&acc)[C::MI][C::NI],
                                           const RowRange& ar, int n0, int wm0, int wn0, int lane) {
  const int n = args.n;
  const bool vec_ok = (n & 3) == 0;
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int row = ar.lo + wm0 + 32 * i + (lane & 31);
    if (row >= ar.end) continue;
    const int64_t rbase = (int64_t)row * n;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
        const float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
        const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (args.c_f32) {
          float* cp = (float*)args.c + rbase + col;
          if (vec_ok && col + 3 < n) {
            *(float4*)cp = make_float4(v0, v1, v2, v3);
          } else {
            if (col + 0 < n) cp[0] = v0;
            if (col + 1 < n) cp[1] = v1;
            if (col + 2 < n) cp[2] = v2;
            if (col + 3 < n) cp[3] = v3;
          }
        } else {
          uint16_t* cp = (uint16_t*)args.c + rbase + col;
          if (vec_ok && col + 3 < n) {
            *(uint2*)cp = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          } else {
            if (col + 0 < n) cp[0] = (uint16_t)f32_to_bf16_bits(v0);
            if (col + 1 < n) cp[1] = (uint16_t)f32_to_bf16_bits(v1);
            if (col + 2 < n) cp[2] = (uint16_t)f32_to_bf16_bits(v2);
            if (col + 3 < n) cp[3] = (uint16_t)f32_to_bf16_bits(v3);
          }
        }
      }
    }
  }
}

// Main loop + epilogue for one output tile.
template <class C, bool KALIGNED>
__device__ __forceinline__ void run_tile(const GemmArgs& args, const uint8_t* b_q, const uint8_t* b_s,
                                         const RowRange& ar, int n0, uint8_t MXFP4_LDS* lds) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (w & 1) * C::WM, wn0 = (w >> 1) * C::WN;
  v16f acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Pointers<C> p;
  make_pointers<C>(p, args.a_q, args.a_s, b_q, b_s, ar, n0, args.n, args.k);
  uint8_t MXFP4_LDS* buf0 = lds;
  uint8_t MXFP4_LDS* buf1 = lds + C::STAGE_BYTES;

  if (KALIGNED) {
    const int nk = args.k / kBK;
    load_stage_dma<C>(buf0, p, 0);
    for (int kt = 0; kt < nk; ++kt) {
      uint8_t MXFP4_LDS* cur = (kt & 1) ? buf1 : buf0;
      uint8_t MXFP4_LDS* nxt = (kt & 1) ? buf0 : buf1;
      if (kt + 1 < nk) {
        load_stage_dma<C>(nxt, p, kt + 1);
        MXFP4_WAIT_VMCNT(C::LOADS);
      } else {
        MXFP4_WAIT_VMCNT(0);
      }
      __syncthreads();
      compute_stage<C>(cur, acc, wm0, wn0, lane);
      __syncthreads();
    }
  } else {
    const int nk = (args.k + kBK - 1) / kBK;
    for (int kt = 0; kt < nk; ++kt) {
      load_stage_generic<C>(buf0, p, kt, args.k);
      __syncthreads();
      compute_stage<C>(buf0, acc, wm0, wn0, lane);
      __syncthreads();
    }
  }
  store_tile<C>(args, acc, ar, n0, wm0, wn0, lane);
}

template <class C, bool KALIGNED>
__global__ __launch_bounds__(kThreads) void gemm_tile_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
  RowRange ar;
  ar.lo = tm * C::BM;
  ar.end = min(ar.lo + C::BM, args.m);
  ar.last = ar.end - 1;
  run_tile<C, KALIGNED>(args, args.b_q, args.b_s, ar, tn * C::BN, (uint8_t MXFP4_LDS*)smem);
}

// Finds the expert owning global m-tile `mt` (m-tiles are counted expert by
// expert, ceil(rows_g / BM) per expert).  Every offset is clamped into
// [0, total_m] and made non-decreasing first, so any offsets give in-range rows.
__device__ __forceinline__ bool find_group(const int32_t* offsets, int groups, int total_m, int bm,
                                           int mt, int& g_out, RowRange& ar) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < groups; base += 64) {
    const int g = base + lane;
    int lo = 0, hi = 0, cnt = 0;
    if (g < groups) {
      lo = min(max(offsets[g], 0), total_m);
      hi = min(max(offsets[g + 1], lo), total_m);
      cnt = (hi - lo + bm - 1) / bm;
    }
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int excl = incl - cnt;
    const bool hit = cnt > 0 && carry + excl <= mt && mt < carry + incl;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll((long long)mask) - 1;
      g_out = __shfl(g, src, 64);
      const int glo = __shfl(lo, src, 64);
      const int ghi = __shfl(hi, src, 64);
      const int first = carry + __shfl(excl, src, 64);
      ar.lo = glo + (mt - first) * bm;
      ar.end = min(ghi, ar.lo + bm);
      ar.last = ar.end - 1;
      return true;
    }
    carry += __shfl(incl, 63, 64);
  }
  return false;
}

template <class C, bool KALIGNED>
__global__ __launch_bounds__(kThreads) void grouped_tile_kernel(GemmArgs args, int mt_bound, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int total = mt_bound * tiles_n;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int mt = t / tiles_n, tn = t - mt * tiles_n;
  int g;
  RowRange ar;
  if (!find_group(args.offsets, args.groups, args.m, C::BM, mt, g, ar)) return;
  const int64_t kb = args.k / 2, ks = args.k / 32;
  const uint8_t* b_q = args.b_q + (int64_t)g * args.n * kb;
  const uint8_t* b_s = args.b_s + (int64_t)g * args.n * ks;
  run_tile<C, KALIGNED>(args, b_q, b_s, ar, tn * C::BN, (uint8_t MXFP4_LDS*)smem);
}

using Cfg256 = TileCfg<256, 256>;
using Cfg128 = TileCfg<128, 128>;

// Dynamic LDS above 64 KiB has to be allowed per kernel.
template <class K>
hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class C>
hipError_t launch_dense(const GemmArgs& args, hipStream_t stream) {
  const int tiles_m = (args.m + C::BM - 1) / C::BM;
  const int tiles_n = (args.n + C::BN - 1) / C::BN;
  const size_t lds = 2 * C::STAGE_BYTES;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (args.k % kBK == 0) {
    hipError_t e = allow_lds(gemm_tile_kernel<C, true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_tile_kernel<C, true>), grid, dim3(kThreads), lds, stream, args, tiles_m, tiles_n);
  } else {
    hipError_t e = allow_lds(gemm_tile_kernel<C, false>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_tile_kernel<C, false>), grid, dim3(kThreads), lds, stream, args, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

template <class C>
hipError_t launch_grouped(const GemmArgs& args, hipStream_t stream) {
  const int mt_bound = (args.m + C::BM - 1) / C::BM + args.groups;
  const int tiles_n = (args.n + C::BN - 1) / C::BN;
  const size_t lds = 2 * C::STAGE_BYTES;
  const dim3 grid((unsigned)(mt_bound * tiles_n));
  if (args.k % kBK == 0) {
    hipError_t e = allow_lds(grouped_tile_kernel<C, true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_tile_kernel<C, true>), grid, dim3(kThreads), lds, stream, args, mt_bound, tiles_n);
  } else {
    hipError_t e = allow_lds(grouped_tile_kernel<C, false>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_tile_kernel<C, false>), grid, dim3(kThreads), lds, stream, args, mt_bound, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tile(const GemmArgs& args, TileKind kind, hipStream_t stream) {
  return kind == kTile256 ? launch_dense<Cfg256>(args, stream) : launch_dense<Cfg128>(args, stream);
}

hipError_t launch_grouped_gemm_tile(const GemmArgs& args, TileKind kind, hipStream_t stream) {
  return kind == kTile256 ? launch_grouped<Cfg256>(args, stream) : launch_grouped<Cfg128>(args, stream);
}

}  // namespace mxfp4
