// NVFP4 on gfx950: quantization and the NT GEMM.
//
// NVFP4 operands ("Packed MXFP4 & NVFP4 GEMM + mega-MoE" page, Summary) are
// packed E2M1 codes with E4M3/UE4M3 scale factors at granularity 16 and a
// global scale, the GEMM result being acc * gs_act * gs_weight; the quadbit
// README ("Accuracy (real models)") keeps the global scale per row (two-level
// NVFP4).  Layout: q [rows, k/2] (element 2j in the low nibble), s [rows, k/16]
// UE4M3 codes, gs [rows] fp32.
//
// Quantization rule (every step an IEEE fp32 operation, so the result is
// reproducible bit for bit): A = max|x| of the row, gs = A / 2688 (1 when
// A == 0); per 16-element block t = amax / (6 * gs), s = t rounded to the
// nearest UE4M3 value (ties to even, saturated at 448), d = s * gs, and each
// code is |x| / d rounded to the nearest E2M1 magnitude (ties to even,
// saturated at 6) with x's sign; a block with d == 0 (s == 0, or s * gs
// underflowing) encodes signed zeros.
//
// The scaled f8f6f4 MFMA of CDNA4 takes E8M0 scales that each cover 32
// elements, so it cannot apply 16-element UE4M3 scales.  The GEMM therefore
// dequantizes instead: e2m1 * ue4m3 has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in BF16.  Each 64-deep K stage of a
// 128x128 tile is loaded packed (16 bytes of codes and 2 scale bytes per
// thread per operand), dequantized once per workgroup into BF16 tiles in LDS
// (the hardware FP4 -> fp32 convert, one multiply, one byte permute) from a
// four-stage register ring of packed loads
// (double-buffered, one barrier per stage), and multiplied on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the epilogue applies
// gs_a[m] * gs_b[n].  This runs at the BF16 MFMA rate (a quarter of FP4's)
// with the dequantization on the vector ALUs.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// quantization
// ---------------------------------------------------------------------------

constexpr int kNvQThreads = 256;

// Nearest UE4M3 value of t >= 0 (ties to the even code), saturated at 448;
// code receives its byte.  The grid spacing is 2^(floor(log2 t) - 3), never
// below the subnormal quantum 2^-9; scaling by a power of two is exact and rint
// rounds half to even.
__device__ __forceinline__ float ue4m3_rne(float t, uint32_t& code) {
  if (!(t > 0.0f)) {
    code = 0;
    return 0.0f;
  }
  if (t >= 448.0f) {
    code = 0x7E;
    return 448.0f;
  }
  const int e = (int)((__float_as_uint(t) >> 23) & 0xFF) - 127;   // fp32 subnormal t gives -127
  const int qexp = max(e - 3, -9);
  const float val = ldexpf(rintf(ldexpf(t, -qexp)), qexp);
  if (val == 0.0f) {
    code = 0;
    return 0.0f;
  }
  const uint32_t vb = __float_as_uint(val);
  const int ev = (int)((vb >> 23) & 0xFF) - 127;
  code = (ev >= -6) ? (uint32_t)(((ev + 7) << 3) | ((vb >> 20) & 7)) : (uint32_t)(val * 512.0f);
  return val;
}

// E2M1 magnitude code of v >= 0: nearest grid value, ties to the even code,
// everything above 5 (including +inf) saturating to code 7 (6.0).
__device__ __forceinline__ uint32_t e2m1_mag(float v) {
  return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) + (uint32_t)(v >= 1.75f) +
         (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) + (uint32_t)(v > 5.0f);
}

__device__ __forceinline__ uint32_t umax16x2(uint32_t a, uint32_t b) {
  return max(a & 0xFFFFu, b & 0xFFFFu) | (max(a >> 16, b >> 16) << 16);
}

__device__ __forceinline__ uint32_t amax8_bits(const uint4& v) {
  const uint32_t m = umax16x2(umax16x2(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                              umax16x2(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
  return max(m & 0xFFFFu, m >> 16);
}

// One workgroup per row; each thread holds SLOTS chunks of 8 elements, and a
// 16-element block is the chunk pair of lanes 2i, 2i + 1.
template <int SLOTS>
__global__ __launch_bounds__(kNvQThreads) void nvfp4_quantize_kernel(const uint4* __restrict__ x, int k,
                                                                    uint32_t* __restrict__ q,
                                                                    uint8_t* __restrict__ scales,
                                                                    float* __restrict__ gs_out) {
  __shared__ uint32_t red[kNvQThreads / 64];
  const int chunks = k >> 3;
  const int64_t rbase = (int64_t)blockIdx.x * chunks;
  uint4 v[SLOTS];
  uint32_t m = 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int c = s * kNvQThreads + threadIdx.x;
    v[s] = make_uint4(0u, 0u, 0u, 0u);
    if (c < chunks) v[s] = x[rbase + c];
    m = max(m, amax8_bits(v[s]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const uint32_t a_bits = max(max(red[0], red[1]), max(red[2], red[3]));
  const float gs = a_bits == 0 ? 1.0f : __uint_as_float(a_bits << 16) / 2688.0f;
  const float six_gs = 6.0f * gs;
  if (threadIdx.x == 0) gs_out[blockIdx.x] = gs;

#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int c = s * kNvQThreads + threadIdx.x;
    if (c >= chunks) continue;   // uniform over each lane pair (chunks is even)
    uint32_t mb = amax8_bits(v[s]);
    mb = max(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0xB1, 0xF, 0xF, true));   // lane ^ 1
    const float t = __uint_as_float(mb << 16) / six_gs;
    uint32_t scode;
    const float sval = ue4m3_rne(t, scode);
    const float d = sval * gs;
    const uint32_t w[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const float mag = __uint_as_float((bits & 0x7FFFu) << 16);
      const uint32_t code = ((bits >> 12) & 8u) | (d == 0.0f ? 0u : e2m1_mag(mag / d));   // d == 0 when s == 0
      packed |= code << (4 * i);
    }
    q[rbase + c] = packed;
    if ((threadIdx.x & 1) == 0) scales[(rbase + c) >> 1] = (uint8_t)scode;
  }
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------

constexpr int kNvBK = 64;                       // K elements per stage
constexpr int kNvPitch = kNvBK * 2 + 16;        // bytes per BF16 LDS row (padded)
constexpr int kNvRing = 4;                      // packed stages in flight per thread

// Square BM x BM output tiles; each of the 2 * BM threads loads and
// dequantizes one 32-element half row of A and one of B per stage.  The waves
// form a WGM x WGN grid, each owning (BM / WGM) x (BM / WGN) in 32 x 32 MFMA
// blocks.
template <int BM_, int WGM_, int WGN_>
struct NvCfg {
  static constexpr int BM = BM_, WGM = WGM_, WGN = WGN_;
  static constexpr int THREADS = 2 * BM;
  static constexpr int MI = BM / WGM / 32, NI = BM / WGN / 32;
  static constexpr int TILE = BM * kNvPitch;    // one operand's BF16 stage
  static constexpr int STAGE = 2 * TILE;        // A then B
  static constexpr int LDS = 2 * STAGE;
  static_assert(WGM * WGN * 64 == THREADS, "one wave per 64 threads");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};
using NvSmall = NvCfg<128, 2, 2>;   // 4 waves of 64 x 64
using NvLarge = NvCfg<256, 2, 4>;   // 8 waves of 128 x 64: half the dequantized elements per flop

typedef float v2f __attribute__((ext_vector_type(2)));

// UE4M3 code -> fp32 value (exact).
__device__ __forceinline__ float ue4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;   // m * 2^-9
}

// 8 codes (one 32-bit word, element 2j in the low nibble of byte j) times a
// scale -> 8 BF16.  The CDNA4 convert turns two E2M1 codes into fp32 (with a
// unit scale every E2M1 value is exact), one fp32 multiply per element applies
// the block scale (exact: at most 6 significant bits), and v_perm keeps the
// upper halves, which are then the BF16 values: two instructions per element.
template <int J>
__device__ __forceinline__ int dequant2(uint32_t word, float s) {
  const v2f p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, J);   // byte J: elements 2J, 2J + 1
  return (int)__builtin_amdgcn_perm(__float_as_uint(p.y * s), __float_as_uint(p.x * s), 0x07060302u);
}

__device__ __forceinline__ v4i dequant8(uint32_t word, float s) {
  return v4i{dequant2<0>(word, s), dequant2<1>(word, s), dequant2<2>(word, s), dequant2<3>(word, s)};
}

struct NvArgs {
  const uint8_t* a_q;  // [m, k/2]
  const uint8_t* a_s;  // [m, k/16]
  const float* a_gs;   // [m]
  const uint8_t* b_q;  // [n, k/2]
  const uint8_t* b_s;  // [n, k/16]
  const float* b_gs;   // [n]
  void* c;             // [m, n]
  int c_f32;
  int m, n, k;
};

// Each thread loads one 32-element half row of a stage per operand: 16 code
// bytes and the 2 scale bytes of its two 16-element blocks.
struct NvLoad {
  uint4 a, b;
  uint32_t as, bs;
};

__device__ __forceinline__ void nv_load(const NvArgs& p, int m0, int n0, int kt, NvLoad& L) {
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t kb = p.k / 2, ks = p.k / 16;
  const int ar = min(m0 + r, p.m - 1), br = min(n0 + r, p.n - 1);
  L.a = *(const uint4*)(p.a_q + ar * kb + kt * (kNvBK / 2) + half * 16);
  L.b = *(const uint4*)(p.b_q + br * kb + kt * (kNvBK / 2) + half * 16);
  L.as = *(const uint16_t*)(p.a_s + ar * ks + kt * (kNvBK / 16) + half * 2);
  L.bs = *(const uint16_t*)(p.b_s + br * ks + kt * (kNvBK / 16) + half * 2);
}

// A thread's dequantized half rows of one stage: 32 BF16 of A and 32 of B.
struct NvDeq {
  v4i a[4], b[4];
};

__device__ __forceinline__ void nv_dequant(const NvLoad& L, NvDeq& D) {
  const uint32_t aw[4] = {L.a.x, L.a.y, L.a.z, L.a.w};
  const uint32_t bw[4] = {L.b.x, L.b.y, L.b.z, L.b.w};
  const float sa0 = ue4m3_value(L.as & 0xFFu), sa1 = ue4m3_value(L.as >> 8);
  const float sb0 = ue4m3_value(L.bs & 0xFFu), sb1 = ue4m3_value(L.bs >> 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    D.a[i] = dequant8(aw[i], i < 2 ? sa0 : sa1);
    D.b[i] = dequant8(bw[i], i < 2 ? sb0 : sb1);
  }
}

template <class C>
__device__ __forceinline__ void nv_write(const NvDeq& D, uint8_t MXFP4_LDS* stage) {
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  uint8_t MXFP4_LDS* arow = stage + r * kNvPitch + half * 64;
  uint8_t MXFP4_LDS* brow = stage + C::TILE + r * kNvPitch + half * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *(v4i MXFP4_LDS*)(arow + 16 * i) = D.a[i];
    *(v4i MXFP4_LDS*)(brow + 16 * i) = D.b[i];
  }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void nvfp4_gemm_kernel(NvArgs p, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t MXFP4_LDS* lds = (uint8_t MXFP4_LDS*)smem;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BM;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (w / C::WGN) * (C::BM / C::WGM), wn0 = (w % C::WGN) * (C::BM / C::WGN);
  const int nk = p.k / kNvBK;

  v16f acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Packed stages go through a ring of four register sets: stage t + 4 is
  // requested while stage t is multiplied, so each load has three stages of
  // MFMAs (and their barriers) to land before it is dequantized into LDS.
  NvLoad L[kNvRing];
#pragma unroll
  for (int u = 0; u < kNvRing; ++u)
    if (u < nk) nv_load(p, m0, n0, u, L[u]);
  {
    NvDeq D0;
    nv_dequant(L[0], D0);
    nv_write<C>(D0, lds);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; kt += kNvRing) {
#pragma unroll
    for (int u = 0; u < kNvRing; ++u) {
      const int t = kt + u;
      if (t >= nk) break;
      if (t + kNvRing < nk) nv_load(p, m0, n0, t + kNvRing, L[u]);   // L[u] held stage t, stored already
      const uint8_t MXFP4_LDS* st = lds + (t & 1) * C::STAGE;
#pragma unroll
      for (int ks = 0; ks < kNvBK / 16; ++ks) {
        const int koff = ks * 32 + (lane >> 5) * 16;       // bytes: 16 K per step, 8 per lane half
        bf16x8_t af[C::MI], bfr[C::NI];
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
          af[i] = *(const bf16x8_t MXFP4_LDS*)(st + (wm0 + 32 * i + (lane & 31)) * kNvPitch + koff);
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
          bfr[j] = *(const bf16x8_t MXFP4_LDS*)(st + C::TILE + (wn0 + 32 * j + (lane & 31)) * kNvPitch + koff);
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
      // the other buffer was last read before the previous barrier
      // the next stage is dequantized after this stage's MFMAs (dequantizing it
      // into registers first raised the register count from 146 to 178 and
      // measured 10 % slower)
      if (t + 1 < nk) {
        NvDeq D;
        nv_dequant(L[(u + 1) % kNvRing], D);
        nv_write<C>(D, lds + ((t + 1) & 1) * C::STAGE);
      }
      __syncthreads();
    }
  }

  // lane l holds output row (l % 32) of each 32-row block and, in register
  // r, column (r / 4) * 8 + (l / 32) * 4 + r % 4 of each 32-column block
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int row = m0 + wm0 + 32 * i + (lane & 31);
    if (row >= p.m) continue;
    const float ga = p.a_gs[row];
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn0 + 32 * j + g * 8 + (lane >> 5) * 4;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cc = min(col + e, p.n - 1);
          o[e] = (acc[i][j][4 * g + e] * ga) * p.b_gs[cc];
        }
        const bool full = col + 3 < p.n && (p.n & 3) == 0;
        if (p.c_f32) {
          float* dst = (float*)p.c + (int64_t)row * p.n + col;
          if (full) {
            *(float4*)dst = make_float4(o[0], o[1], o[2], o[3]);
          } else {
            for (int e = 0; e < 4; ++e)
              if (col + e < p.n) dst[e] = o[e];
          }
        } else {
          uint16_t* dst = (uint16_t*)p.c + (int64_t)row * p.n + col;
          if (full) {
            *(uint2*)dst = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          } else {
            for (int e = 0; e < 4; ++e)
              if (col + e < p.n) dst[e] = (uint16_t)f32_to_bf16_bits(o[e]);
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_nvfp4_quantize(const void* x, int rows, int k, void* q, void* scales, float* gs,
                                 hipStream_t stream) {
  if (!grid_fits(rows, kNvQThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)rows), block(kNvQThreads);
  if (k <= 2 * 8 * kNvQThreads)
    hipLaunchKernelGGL(nvfp4_quantize_kernel<2>, grid, block, 0, stream, (const uint4*)x, k, (uint32_t*)q,
                       (uint8_t*)scales, gs);
  else if (k <= 4 * 8 * kNvQThreads)
    hipLaunchKernelGGL(nvfp4_quantize_kernel<4>, grid, block, 0, stream, (const uint4*)x, k, (uint32_t*)q,
                       (uint8_t*)scales, gs);
  else
    hipLaunchKernelGGL(nvfp4_quantize_kernel<kNormMaxSlots>, grid, block, 0, stream, (const uint4*)x, k,
                       (uint32_t*)q, (uint8_t*)scales, gs);
  return hipGetLastError();
}

template <class C>
hipError_t launch_nv_cfg(const NvArgs& p, hipStream_t stream) {
  const int tiles_m = (p.m + C::BM - 1) / C::BM, tiles_n = (p.n + C::BM - 1) / C::BM;
  const int64_t blocks = (int64_t)tiles_m * tiles_n;
  if (!grid_fits(blocks, C::THREADS)) return hipErrorInvalidConfiguration;
  hipError_t e = hipFuncSetAttribute((const void*)nvfp4_gemm_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nvfp4_gemm_kernel<C>, dim3((unsigned)blocks), dim3(C::THREADS), C::LDS, stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

// 256 x 256 tiles once they fill the chip (256 tiles), 128 x 128 below that.
hipError_t launch_nvfp4_gemm(const void* a_q, const void* a_s, const float* a_gs, const void* b_q, const void* b_s,
                             const float* b_gs, void* c, bool c_f32, int m, int n, int k, hipStream_t stream) {
  NvArgs p{(const uint8_t*)a_q, (const uint8_t*)a_s, a_gs, (const uint8_t*)b_q, (const uint8_t*)b_s, b_gs,
           c, c_f32 ? 1 : 0, m, n, k};
  const int64_t large_tiles = (int64_t)((m + 255) / 256) * ((n + 255) / 256);
  if (large_tiles >= 256) return launch_nv_cfg<NvLarge>(p, stream);
  return launch_nv_cfg<NvSmall>(p, stream);
}

}  // namespace mxfp4
