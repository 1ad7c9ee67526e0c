// Small-M block-scaled FP4 GEMM that streams the weight matrix (gfx950).
//
// Same operation as the tile kernels, C[m][n] = sum_k A[m][k] * B[n][k] over
// MXFP4 operands ("Packed MXFP4 & NVFP4 GEMM + mega-MoE" page, Summary:
// mxfp4_gemm_nt; its decode shapes are the small-M case), for M up to a few
// hundred rows.  There B (the weights, N x K) is read once from HBM and A is
// small and shared by every workgroup, so the kernel is laid out for bandwidth:
//
//  * One workgroup per 64 output columns of one (32*MB)-row M tile, over the
//    whole K: B is read exactly once and no cross-workgroup reduction exists.
//  * The copy unit is a "pair": 512 K elements = two 256-K stages of 128 code
//    bytes per row (A rows then B rows, the tile kernels' conflict-free
//    128-byte swizzled row layout) plus the 16 scale bytes of every row.
//    Every copy is global_load_lds_dwordx4 straight into LDS, 8 whole 128-byte
//    row pieces per wave instruction.  NP pair buffers form a ring; NP - 1 pairs
//    are in flight while one is consumed.  Both operands go through LDS:
//    loads straight into registers in the MFMA operand layout touch 32 rows
//    per instruction and measured far slower on this path than whole-row
//    copies.  A short kernel like this one is bound by the bytes each CU keeps
//    in flight (delivery ~ bytes in flight / loaded latency), which the LDS
//    ring caps; A's share of the ring is what limits larger M.
//  * The 4 waves split each 256-K stage by k-step: wave w computes k-step w
//    (K elements 64w..64w+63 of the stage) for the whole 32*MB x 64 tile, so
//    every code byte copied into LDS is read by exactly one wave.  At the end
//    the four fp32 partial tiles are reduce-scattered through LDS, each output
//    summed in the fixed order wave 0 + wave 1 + wave 2 + wave 3, so results
//    do not depend on timing.  BF16 results are gathered into a row-major
//    tile in LDS and leave as whole 128-byte rows in 16-byte stores.
//  * MFMA operands as in the tile kernels: v_mfma_scale_f32_32x32x64_f8f6f4,
//    FP4 on both sides, B fed as the first operand so lane l holds output row
//    l % 32 and runs of four consecutive columns.
//
// W4A8 (MXFP8 activations): A rows carry one code byte per element, 256 bytes
// per stage in sixteen chunks at c ^ (r & 15), and the MFMA takes A as an FP8
// operand (lane half h holds K [16h, 16h + 16) and [32 + 16h, 48 + 16h) of its
// k-step).  Doubling A's share of the ring limits the M tile to 64 rows; for
// M up to 128 the two M tiles of one 64-column slice are dispatched next to
// each other on the same XCD, so the second reads the weight slice from that
// XCD's L2 rather than HBM.
//
// Requirements (checked by the host): k % 512 == 0 and 16-byte aligned scale
// arrays.  Rows past M and columns past N read a clamped valid row and are
// never stored.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;    // code bytes per row per 256-K stage
// Cache policy of the weight loads and copies: non-temporal.  The weight is
// read once per launch; streaming it past the caches leaves the L2 to the
// activation, which every workgroup re-reads.  Same-box A/B: 4 % faster for
// the prepacked decode GEMM, 1.5-2.5 % for this streaming kernel.
constexpr int kLoadNT = 2;
constexpr int kBN = 64;
// Split-K workspace of the both-prepacked kernel: the arrival counters fill a
// fixed region at the start (so one zeroed workspace serves every shape), the
// partial tiles follow.
constexpr size_t kPPCounterBytes = 65536;
constexpr int kPPMaxTiles = (int)(kPPCounterBytes / sizeof(int));

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int MB_, int NP_, bool A8_ = false, bool PRE_ = false>
struct StreamCfg {
  static constexpr int MB = MB_, NP = NP_;
  static constexpr bool A8 = A8_;                          // A in FP8 E4M3 (W4A8)
  static constexpr bool PRE = PRE_;                        // B prepacked, loaded into registers
  static constexpr int BM = 32 * MB;
  static constexpr int B_LDS_ROWS = PRE ? 0 : kBN;         // B rows staged in LDS
  static constexpr int ROWS = BM + B_LDS_ROWS;             // A rows, then B rows
  static constexpr int A_ROW = A8 ? 2 * kRowBytes : kRowBytes;
  static constexpr int A_SHIFT = A8 ? 4 : 3;               // log2 of the 16-byte chunks in an A row
  static constexpr int A_BYTES = BM * A_ROW;
  static constexpr int A_SLOTS = A_BYTES / 16;
  static constexpr int STAGE = A_BYTES + B_LDS_ROWS * kRowBytes;
  static constexpr int SCALES = kThreads * 16;            // one 16-byte piece per thread (rows >= ROWS: padding)
  static constexpr int PAIR = 2 * STAGE + SCALES;
  static constexpr int CODE_LOADS = STAGE / 16 / kThreads;  // 16-byte copies per thread per stage
  static constexpr int PAIR_LOADS = 2 * CODE_LOADS + 1;   // vector-memory ops per thread per pair
  static constexpr int XCH = 4 * MB * 8 * 64 * 16;        // reduce-scatter exchange: 4 waves x all units
  static constexpr int C_PITCH = kBN * 2 + 16;             // bf16 output tile row, padded
  static constexpr int C_TILE = BM * C_PITCH;              // placed after the exchange area
  static constexpr int LDS = (NP * PAIR > XCH + C_TILE) ? NP * PAIR : XCH + C_TILE;
  static_assert(STAGE % (16 * kThreads) == 0, "code copies must split evenly over the threads");
  static_assert(A_SLOTS % 64 == 0, "a wave's copy instruction lies wholly in A or in B");
  static_assert(ROWS <= (PRE ? 3 * 64 : kThreads), "one scale piece per row (prepacked B: wave 3 copies B's scales)");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((NP - 2) * PAIR_LOADS <= 63, "vmcnt range");
};

// Per-thread copy sources.  Copy j of a stage moves slot (j*4 + wave)*64 + lane:
// A slots first (row slot / chunks-per-row, logical chunk (slot % chunks) ^ the
// row's swizzle), then B slots; pointers are at pair 0.
template <class C>
struct Sources {
  const uint8_t* code[C::CODE_LOADS];
  const uint8_t* scale;
};

template <class C>
__device__ __forceinline__ void make_sources(Sources<C>& src, const GemmArgs& args, int m0, int n0) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t kb = args.k / 2, ks = args.k / 32, ka = C::A8 ? args.k : kb;
#pragma unroll
  for (int j = 0; j < C::CODE_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    if (slot < C::A_SLOTS) {
      const int r = slot >> C::A_SHIFT;
      const int lc = (slot & ((1 << C::A_SHIFT) - 1)) ^ (C::A8 ? (r & 15) : swz(r));
      src.code[j] = args.a_q + min(m0 + r, args.m - 1) * ka + lc * 16;
    } else {
      const int bs = slot - C::A_SLOTS;
      const int r = bs >> 3, lc = (bs & 7) ^ swz(r);
      src.code[j] = args.b_q + min(n0 + r, args.n - 1) * kb + lc * 16;
    }
  }
  const int r = threadIdx.x;   // padding rows re-read A's row m0 into the unused pieces
  src.scale = (r < C::BM || r >= C::ROWS) ? args.a_s + min(m0 + (r < C::BM ? r : 0), args.m - 1) * ks
                                          : args.b_s + min(n0 + r - C::BM, args.n - 1) * ks;
}

// All copies of pair p into `buf` (stage 2p, stage 2p+1, then the scale pieces).
template <class C>
__device__ __forceinline__ void copy_pair(uint8_t MXFP4_LDS* buf, const Sources<C>& src, int p) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // LDS base must be wave-uniform (M0)
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < C::CODE_LOADS; ++j) {
      // wave-uniform: A_SLOTS is a multiple of 64
      if ((j * 4 + w) * 64 < C::A_SLOTS)
        g2lds_16(src.code[j] + (2 * p + s) * C::A_ROW,
                 (MXFP4_LDS void*)(buf + s * C::STAGE + (j * 4 + w) * 64 * 16));
      else   // weight rows: read once per launch, streamed past the caches (non-temporal)
        __builtin_amdgcn_global_load_lds(src.code[j] + (2 * p + s) * kRowBytes,
                                         (MXFP4_LDS void*)(buf + s * C::STAGE + (j * 4 + w) * 64 * 16), 16, 0,
                                         kLoadNT);
    }
  g2lds_16(src.scale + p * 16, (MXFP4_LDS void*)(buf + 2 * C::STAGE + w * 64 * 16));
}

// Wait until at most `pairs` pairs of this thread's copies are outstanding.
template <class C>
__device__ __forceinline__ void wait_pairs(int pairs) {
  switch (pairs) {
    case 0: MXFP4_WAIT_VMCNT(0); break;
    case 1: MXFP4_WAIT_VMCNT(C::PAIR_LOADS); break;
    case 2: MXFP4_WAIT_VMCNT(2 * C::PAIR_LOADS); break;
    default: MXFP4_WAIT_VMCNT(3 * C::PAIR_LOADS); break;
  }
}

__device__ __forceinline__ void barrier_lds() {
  MXFP4_WAIT_LGKM0();
  asm volatile("s_barrier" ::: "memory");
}

// Fragments and scale bytes of one wave's k-step of one stage.
template <class C>
struct Step {
  typename std::conditional<C::A8, v8i, v4i>::type a[C::MB];
  v4i b[2];
  int sa[C::MB];
  int sb[2];
};

template <class C>
__device__ __forceinline__ void read_step(const uint8_t MXFP4_LDS* buf, int s, int w, int lane, Step<C>& st) {
  const uint8_t MXFP4_LDS* stage = buf + s * C::STAGE;
  const uint8_t MXFP4_LDS* scales = buf + 2 * C::STAGE + 8 * s + 2 * w + (lane >> 5);
  const int c = 2 * w + (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    const int r = 32 * i + (lane & 31);
    if constexpr (C::A8) {
      // FP8 fragment of k-step w: chunks 4w + h and 4w + 2 + h (h = lane half)
      const int h = lane >> 5;
      const v4i lo = *(const v4i MXFP4_LDS*)(stage + r * C::A_ROW + (((4 * w + h) ^ (r & 15)) << 4));
      const v4i hi = *(const v4i MXFP4_LDS*)(stage + r * C::A_ROW + (((4 * w + 2 + h) ^ (r & 15)) << 4));
      st.a[i] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    } else {
      st.a[i] = *(const v4i MXFP4_LDS*)(stage + r * kRowBytes + ((c ^ swz(r)) << 4));
    }
    st.sa[i] = scales[r * 16];
  }
  if constexpr (!C::PRE) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 32 * j + (lane & 31);
      st.b[j] = *(const v4i MXFP4_LDS*)(stage + C::A_BYTES + r * kRowBytes + ((c ^ swz(r)) << 4));
      st.sb[j] = scales[(C::BM + r) * 16];
    }
  }
}

template <class C>
__device__ __forceinline__ void mma_step(const Step<C>& st, v16f (&acc)[C::MB][2]) {
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (C::A8)
        acc[i][j] = mfma32_fp4_fp8<0>(st.b[j], st.a[i], acc[i][j], st.sb[j], st.sa[i]);
      else
        acc[i][j] = mfma32_fp4<0>(st.b[j], st.a[i], acc[i][j], st.sb[j], st.sa[i]);
    }
}

// Workgroup -> (M tile, 64-column slice).  Workgroups go to the 8 XCDs round
// robin (b % 8), so in every run of 8 * tiles_m workgroups the M tiles of one
// slice share an XCD (its L2 serves the slice's weights to all but the first)
// and are dispatched close together; workgroups past the last slice exit.
__device__ __forceinline__ bool stream_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int run = 8 * tiles_m;
  const int g = b / run, r = b - g * run;
  tm = r >> 3;
  tn = g * 8 + (r & 7);
  return tn < tiles_n;
}

// Reduce-scatter of the four waves' fp32 partial tiles.  The accumulators
// split into U units of 64 lanes x 4 floats (row block i, column block j,
// column group q); wave w owns units [w*U/4, (w+1)*U/4).  Each wave parks the
// units it does not own in LDS, then sums each of its units over the waves in
// the fixed order 0, 1, 2, 3 into own[] (own[t] is unit w*U/4 + t).
template <class C>
__device__ __forceinline__ void reduce_units(const v16f (&acc)[C::MB][2], uint8_t MXFP4_LDS* lds, int w, int lane,
                                             v4f (&own)[C::MB * 2]) {
  constexpr int U = C::MB * 8, UW = U / 4;
  v4f MXFP4_LDS* xch = (v4f MXFP4_LDS*)lds;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = u / 8, j = (u / 4) % 2, q = u % 4;
    if (u / UW != w) {
      v4f v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      xch[(w * U + u) * 64 + lane] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u / UW != w) continue;   // wave-uniform
    const int i = u / 8, j = (u / 4) % 2, q = u % 4;
    const v4f mine = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    v4f v = (w == 0) ? mine : xch[u * 64 + lane];
#pragma unroll
    for (int src = 1; src < 4; ++src) v += (w == src) ? mine : xch[(src * U + u) * 64 + lane];
    own[u % UW] = v;
  }
}

// The stores of C from each wave's summed units (reduce_units).
template <class C>
__device__ __forceinline__ void store_units(const v4f (&own)[C::MB * 2], const GemmArgs& args, int m0, int n0,
                                            uint8_t MXFP4_LDS* lds, int w, int lane) {
  constexpr int U = C::MB * 8, UW = U / 4;
  const int rows = min(C::BM, args.m - m0);
  const int cols = min(kBN, args.n - n0);
  const int n = args.n;
  if (!args.c_f32) {
    // BF16: the summed units go into a row-major tile in LDS, then whole
    // 128-byte output rows leave in 16-byte non-temporal stores (8-byte stores
    // scattered over 32 rows measured far slower in the tile kernels).
    uint8_t MXFP4_LDS* ctile = lds + C::XCH;
#pragma unroll
    for (int t = 0; t < UW; ++t) {
      const int u = w * UW + t;
      const int i = u / 8, j = (u / 4) % 2, q = u % 4;
      const v4f v = own[t];
      const int r = 32 * i + (lane & 31);
      const int col = 32 * j + 8 * q + 4 * (lane >> 5);
      bf16x2_t lo = {(__bf16)v.x, (__bf16)v.y};
      bf16x2_t hi = {(__bf16)v.z, (__bf16)v.w};
      v2i pk = {__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
      *(v2i MXFP4_LDS*)(ctile + r * C::C_PITCH + col * 2) = pk;
    }
    __syncthreads();
    const bool vec_ok = (n & 7) == 0;   // 16-byte aligned output rows
    for (int idx = threadIdx.x; idx < rows * 8; idx += kThreads) {
      const int r = idx >> 3, cc = idx & 7;
      const int col = cc * 8;
      if (col >= cols) continue;
      const v4i v = *(const v4i MXFP4_LDS*)(ctile + r * C::C_PITCH + cc * 16);
      uint16_t* dst = (uint16_t*)args.c + (int64_t)(m0 + r) * n + n0 + col;
      const int cnt = min(8, cols - col);
      if (vec_ok && cnt == 8) {
        __builtin_nontemporal_store(v, (v4i*)dst);
      } else {
        for (int e = 0; e < cnt; ++e) {
          const uint32_t word = (uint32_t)((e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w);
          dst[e] = (uint16_t)(word >> (16 * (e & 1)));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < UW; ++t) {
    const int u = w * UW + t;
    const int i = u / 8, j = (u / 4) % 2, q = u % 4;
    const v4f v = own[t];
    const int r = 32 * i + (lane & 31);
    const int col = 32 * j + 8 * q + 4 * (lane >> 5);
    const int cnt = min(4, cols - col);
    if (r >= rows || cnt <= 0) continue;
    float* dst = (float*)args.c + (int64_t)(m0 + r) * n + n0 + col;
    if (cnt == 4 && (n & 3) == 0) {
      *(v4f*)dst = v;
    } else {
      for (int e = 0; e < cnt; ++e) dst[e] = v[e];
    }
  }
}

// Reduction of the four waves' partial tiles and the stores of C.
template <class C>
__device__ __forceinline__ void stream_epilogue(v16f (&acc)[C::MB][2], const GemmArgs& args, int m0, int n0,
                                                uint8_t MXFP4_LDS* lds, int w, int lane) {
  v4f own[C::MB * 2];
  reduce_units<C>(acc, lds, w, lane, own);
  store_units<C>(own, args, m0, n0, lds, w, lane);
}

template <class C>
__global__ __launch_bounds__(kThreads) void gemm_stream_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t MXFP4_LDS* lds = (uint8_t MXFP4_LDS*)smem;
  int tm, tn;
  if (!stream_coords(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  const int m0 = tm * C::BM, n0 = tn * kBN;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;

  v16f acc[C::MB][2];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Sources<C> src;
  make_sources<C>(src, args, m0, n0);
  const int np = args.k / 512;
  for (int p = 0; p < C::NP - 1 && p < np; ++p) copy_pair<C>(lds + p * C::PAIR, src, p);

  int slot = 0;                 // ring buffer of pair p
  for (int p = 0; p < np; ++p) {
    // pair p has landed for this thread; the pairs issued after it may still fly
    wait_pairs<C>(min(C::NP - 2, np - 1 - p));
    // ... and for every thread; every wave has also finished reading pair p - 1
    barrier_lds();
    if (p + C::NP - 1 < np) {
      const int refill = (slot == 0) ? C::NP - 1 : slot - 1;   // buffer of pair p - 1
      copy_pair<C>(lds + refill * C::PAIR, src, p + C::NP - 1);
    }
    const uint8_t MXFP4_LDS* buf = lds + slot * C::PAIR;
    Step<C> s0, s1;
    read_step<C>(buf, 0, w, lane, s0);
    read_step<C>(buf, 1, w, lane, s1);
    mma_step<C>(s0, acc);
    mma_step<C>(s1, acc);
    slot = (slot + 1 == C::NP) ? 0 : slot + 1;
  }
  MXFP4_WAIT_VMCNT(0);
  __syncthreads();   // every wave is done with the ring

  stream_epilogue<C>(acc, args, m0, n0, lds, w, lane);
}

template <class C>
hipError_t launch_cfg(const GemmArgs& args, hipStream_t stream) {
  const auto kernel = gemm_stream_kernel<C>;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  const int tiles_n = (args.n + kBN - 1) / kBN;
  const int tiles_m = (args.m + C::BM - 1) / C::BM;
  const int64_t blocks = (int64_t)tiles_m * ((tiles_n + 7) / 8) * 8;   // whole runs of 8 * tiles_m
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), C::LDS, stream, args, tiles_m, tiles_n);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Prepacked weights.  A weight matrix is quantized once, so its layout in HBM
// is free: the prepacked form stores, for every 64-row panel of B and every
// 512-K pair, the exact bytes each lane of each wave feeds the MFMA, so a wave
// loads B straight into registers with whole 1 KB contiguous reads and B needs
// no LDS at all.  Per (panel, pair):
//   codes, 16 KB: byte w*4096 + u*1024 + l*16 + c, u = 2s + j, is code byte c
//     of row 64*panel + 32j + (l % 32) at row byte 256*pair + 128s + 32w +
//     16*(l / 32) (wave w's k-step of stage s, column block j, lane l);
//   scales, 1 KB: byte w*256 + l*4 + (2s + j) is the scale of that row for
//     the 32-element block 16*pair + 8s + 2w + l / 32.
// Rows past N are zero codes with scale byte 0.  Panels are stored in order,
// pairs in order within a panel.
constexpr int kPreCodeBlock = 16 * 1024;
constexpr int kPreScaleBlock = 1024;
constexpr int kPreDepth = 4;   // B pairs in each wave's register ring (depths 4-8 measured within 2 %)
constexpr int kPreBLoads = 4;  // vector-memory ops per B pair per thread

__global__ __launch_bounds__(kThreads) void prepack_kernel(const uint8_t* __restrict__ b_q,
                                                           const uint8_t* __restrict__ b_s, int n, int k,
                                                           uint8_t* __restrict__ bp_q, uint8_t* __restrict__ bp_s) {
  const int np = k / 512;
  const int64_t blk = blockIdx.x;                    // panel * np + pair
  const int panel = (int)(blk / np), p = (int)(blk - (int64_t)panel * np);
  const int64_t kb = k / 2, ks = k / 32;
  for (int c = threadIdx.x; c < kPreCodeBlock / 16; c += kThreads) {
    const int w = c >> 8, u = (c >> 6) & 3, l = c & 63;
    const int s = u >> 1, j = u & 1;
    const int row = panel * kBN + 32 * j + (l & 31);
    v4i v = {0, 0, 0, 0};
    if (row < n) v = *(const v4i*)(b_q + row * kb + 256 * p + 128 * s + 32 * w + 16 * (l >> 5));
    *(v4i*)(bp_q + blk * kPreCodeBlock + c * 16) = v;
  }
  const int d = threadIdx.x, w = d >> 6, l = d & 63;   // one scale word per thread
  uint32_t word = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int s = b >> 1, j = b & 1;
    const int row = panel * kBN + 32 * j + (l & 31);
    if (row < n) word |= (uint32_t)b_s[row * ks + 16 * p + 8 * s + 2 * w + (l >> 5)] << (8 * b);
  }
  *(uint32_t*)(bp_s + blk * kPreScaleBlock + d * 4) = word;
}

// A's copies in the prepacked kernel: buffer_load ... lds (MUBUF) rather than
// global_load_lds.  The latter is a FLAT-encoded instruction that also writes
// LDS, and while one is outstanding the compiler takes the vector-memory
// counter to be out of order and waits for zero before any use of a register
// loaded from memory, which would drain the whole B ring.  Buffer copies keep
// every vector-memory op in one in-order class.  Offsets past a resource's
// bytes read zeros, so no copy can leave the tile's A rows or the panel.
//   code copies: resource over A rows [m0, m0 + rows), per-thread voffset of
//                its row and chunk, soffset = the 128-byte stage step;
//   scale pieces: waves 0-2 copy A rows' 16-byte pieces (rows past the tile
//                 re-read its first row), wave 3 copies the panel's prepacked
//                 B scale block (1 KB per pair), landing at LDS byte 3072 of
//                 the pair's scale area.
template <class C>
struct PreCopies {
  __amdgpu_buffer_rsrc_t code;
  __amdgpu_buffer_rsrc_t scale;   // wave-uniform: A scales (waves 0-2) or B's prepacked scales (wave 3)
  uint32_t code_off[C::CODE_LOADS];
  uint32_t scale_off;
  uint32_t scale_step;            // bytes per pair in the scale resource
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  return make_rsrc((const void*)(uintptr_t)u, bytes);
}

template <class C>
__device__ __forceinline__ void make_pre_copies(PreCopies<C>& cp, const GemmArgs& args, int m0, int tn, int np,
                                                int w, int lane) {
  const int ka = C::A8 ? args.k : args.k / 2, ks = args.k / 32;   // A bytes per row
  const int rows = min(C::BM, args.m - m0);
  cp.code = uniform_rsrc(args.a_q + (int64_t)m0 * ka, (uint32_t)rows * ka);
#pragma unroll
  for (int j = 0; j < C::CODE_LOADS; ++j) {
    const int slot = (j * 4 + w) * 64 + lane;
    const int r = slot >> C::A_SHIFT;
    const int lc = (slot & ((1 << C::A_SHIFT) - 1)) ^ (C::A8 ? (r & 15) : swz(r));
    cp.code_off[j] = (uint32_t)min(r, rows - 1) * ka + lc * 16;
  }
  if (w == 3) {
    cp.scale = uniform_rsrc(args.b_s + (int64_t)tn * np * kPreScaleBlock, (uint32_t)np * kPreScaleBlock);
    cp.scale_off = lane * 16;
    cp.scale_step = kPreScaleBlock;
  } else {
    cp.scale = uniform_rsrc(args.a_s + (int64_t)m0 * ks, (uint32_t)rows * ks);
    const int r = w * 64 + lane;
    cp.scale_off = (uint32_t)(r < rows ? r : 0) * ks;
    cp.scale_step = 16;
  }
}

template <class C>
__device__ __forceinline__ void copy_pair_pre(uint8_t MXFP4_LDS* buf, const PreCopies<C>& cp, int p, int w) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < C::CODE_LOADS; ++j)
      buf2lds_16(cp.code, cp.code_off[j], (uint32_t)(2 * p + s) * C::A_ROW,
                 (MXFP4_LDS void*)(buf + s * C::STAGE + (j * 4 + w) * 64 * 16));
  buf2lds_16(cp.scale, cp.scale_off, (uint32_t)p * cp.scale_step, (MXFP4_LDS void*)(buf + 2 * C::STAGE + w * 64 * 16));
}

// One wave's B operands of one pair: q[2s + j] feeds stage s, column block j.
struct BPair {
  v4i q[4];
};

// The four 1 KB loads of pair p.  The pair's offset goes in the per-lane
// offset, which the buffer's range check covers, so a pair past the panel's
// last one reads zeros without touching memory.  The empty asm statements keep
// these loads and the LDS copies in program order, which the vmcnt arithmetic
// counts on.
__device__ __forceinline__ void load_bpair(BPair& b, __amdgpu_buffer_rsrc_t r, uint32_t voff, int p) {
  asm volatile("" ::: "memory");
  const uint32_t off = voff + (uint32_t)p * kPreCodeBlock;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    b.q[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off + u * 1024, 0, kLoadNT));
  asm volatile("" ::: "memory");
}

// Issue order: a prologue of steps q = 0 .. D-2, each [A pair q if q <= NP-2]
// [B pair q], then in iteration t [A pair t+NP-1 if it exists][B pair t+D-1].
// Prologue A copies past the last pair re-copy the last pair (only when
// K < 512 * (NP - 1)).  Loads past the last B pair fall outside the panel's
// buffer and return zeros without touching memory; the runtime-K loop issues
// them so that no path through it skips a load (which keeps the compiler's
// own waits for the B registers tight), but their results are never used and
// the compiler may delete them.  Loads complete in order, so "A pair p has
// landed" is "at most the ops issued after it are outstanding".  This counts
// those ops at the top of iteration p, leaving out every B load past the last
// pair: if such a load was issued, the wait is only stricter than needed.
// At most NP - 1 A pairs and D - 1 B pairs are ever outstanding, which keeps
// the count inside the counter's range (< 64).
template <class C>
__host__ __device__ constexpr int pre_ops_after_a(int p, int np) {
  constexpr int LA = C::PAIR_LOADS, LB = kPreBLoads, NP = C::NP, D = kPreDepth;
  int cnt = 0, t = 0;
  if (p <= NP - 2) {
    cnt += LB;           // B pair p follows A pair p in prologue step p
    for (int q = p + 1; q <= D - 2; ++q) cnt += (q <= NP - 2 ? LA : 0) + (q < np ? LB : 0);
  } else {
    const int t0 = p - NP + 1;   // the iteration that issued A pair p
    cnt += (t0 + D - 1 < np) ? LB : 0;
    t = t0 + 1;
  }
  for (; t < p; ++t) cnt += ((t + NP - 1 < np) ? LA : 0) + ((t + D - 1 < np) ? LB : 0);
  return cnt;
}

#define MXFP4_VM_CASE(n) \
  case n:                \
    MXFP4_WAIT_VMCNT(n); \
    break;
#define MXFP4_VM_CASE8(n) \
  MXFP4_VM_CASE(n) MXFP4_VM_CASE(n + 1) MXFP4_VM_CASE(n + 2) MXFP4_VM_CASE(n + 3) \
  MXFP4_VM_CASE(n + 4) MXFP4_VM_CASE(n + 5) MXFP4_VM_CASE(n + 6) MXFP4_VM_CASE(n + 7)

// s_waitcnt takes an immediate: dispatch a wave-uniform count to it.
__device__ __forceinline__ void wait_vm_at_most(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
    MXFP4_VM_CASE8(0) MXFP4_VM_CASE8(8) MXFP4_VM_CASE8(16) MXFP4_VM_CASE8(24)
    MXFP4_VM_CASE8(32) MXFP4_VM_CASE8(40) MXFP4_VM_CASE8(48) MXFP4_VM_CASE8(56)
    default: MXFP4_WAIT_VMCNT(0); break;
  }
}
#undef MXFP4_VM_CASE8
#undef MXFP4_VM_CASE

// The 32x32x64 block-scaled FP4 MFMA with the scale byte selected separately
// for the two operands (OPSEL_A picks a byte of sa, OPSEL_B a byte of sb).
template <int OPSEL_A, int OPSEL_B>
__device__ __forceinline__ v16f mfma32_fp4_sel(v4i a, v4i b, v16f acc, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc, kMfmaFmtFp4, kMfmaFmtFp4,
                                                         OPSEL_A, sa, OPSEL_B, sb);
}

// The same with the second operand in FP8 E4M3 (W4A8: 32 codes per lane, as
// mfma32_fp4_fp8).
template <int OPSEL_A, int OPSEL_B>
__device__ __forceinline__ v16f mfma32_fp4_fp8_sel(v4i a, v8i b, v16f acc, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, acc, kMfmaFmtFp4, kMfmaFmtFp8,
                                                         OPSEL_A, sa, OPSEL_B, sb);
}

template <class C, int S>
__device__ __forceinline__ void mma_pre(const Step<C>& st, const BPair& b, int bsc, v16f (&acc)[C::MB][2]) {
#pragma unroll
  for (int i = 0; i < C::MB; ++i) {
    if constexpr (C::A8) {
      acc[i][0] = mfma32_fp4_fp8_sel<2 * S, 0>(b.q[2 * S], st.a[i], acc[i][0], bsc, st.sa[i]);
      acc[i][1] = mfma32_fp4_fp8_sel<2 * S + 1, 0>(b.q[2 * S + 1], st.a[i], acc[i][1], bsc, st.sa[i]);
    } else {
      acc[i][0] = mfma32_fp4_sel<2 * S, 0>(b.q[2 * S], st.a[i], acc[i][0], bsc, st.sa[i]);
      acc[i][1] = mfma32_fp4_sel<2 * S + 1, 0>(b.q[2 * S + 1], st.a[i], acc[i][1], bsc, st.sa[i]);
    }
  }
}

// One pair of the prepacked-B pipeline (pair p of a chunk of np pairs that
// starts at pair p0 of the panel; B pair p in `cur`; the ring slot of pair
// p - 1 refilled with pair p + kPreDepth - 1).
template <class C>
__device__ __forceinline__ void pre_pair(uint8_t MXFP4_LDS* lds, const PreCopies<C>& src, int p0, int p, int np,
                                         int& slot, const BPair& cur, BPair& refill_b, __amdgpu_buffer_rsrc_t rb,
                                         uint32_t voff, int w, int lane, v16f (&acc)[C::MB][2]) {
  barrier_lds();                // A pair p is in LDS for every wave; pair p - 1 is read
  if (p + C::NP - 1 < np) {
    const int refill = (slot == 0) ? C::NP - 1 : slot - 1;   // buffer of pair p - 1
    copy_pair_pre<C>(lds + refill * C::PAIR, src, p0 + p + C::NP - 1, w);
  }
  if (p + kPreDepth - 1 < np) load_bpair(refill_b, rb, voff, p0 + p + kPreDepth - 1);
  const uint8_t MXFP4_LDS* buf = lds + slot * C::PAIR;
  const int bsc = *(const int MXFP4_LDS*)(buf + 2 * C::STAGE + 3 * 64 * 16 + w * 256 + lane * 4);
  Step<C> s0, s1;
  read_step<C>(buf, 0, w, lane, s0);
  read_step<C>(buf, 1, w, lane, s1);
  mma_pre<C, 0>(s0, cur, bsc, acc);
  mma_pre<C, 1>(s1, cur, bsc, acc);
  slot = (slot + 1 == C::NP) ? 0 : slot + 1;
}

// CH pairs starting at pair p0 as straight-line code: the A ring in LDS and
// the B ring in registers both start empty and drain within the chunk, so ring
// slots and wait counts are constants and no register crosses a loop back-edge
// (a B ring carried round a runtime-K loop made the compiler copy it across
// the back-edge and spill).  The barrier first: the previous chunk's waves may
// still read the LDS slots this chunk's first copies overwrite.
template <class C, int CH>
__device__ __forceinline__ void pre_chunk(uint8_t MXFP4_LDS* lds, const PreCopies<C>& src, int p0,
                                          __amdgpu_buffer_rsrc_t rb, uint32_t voff, int w, int lane,
                                          v16f (&acc)[C::MB][2]) {
  barrier_lds();
  BPair ring[kPreDepth];
#pragma unroll
  for (int q = 0; q < kPreDepth - 1; ++q) {
    if (q <= C::NP - 2) copy_pair_pre<C>(lds + q * C::PAIR, src, p0 + min(q, CH - 1), w);
    if (q < CH) load_bpair(ring[q], rb, voff, p0 + q);
  }
  int slot = 0;                 // LDS ring buffer of A pair p
#pragma unroll
  for (int p = 0; p < CH; ++p) {   // B pair p sits in ring[p % kPreDepth]
    wait_vm_at_most(pre_ops_after_a<C>(p, CH));   // a constant once unrolled
    pre_pair<C>(lds, src, p0, p, CH, slot, ring[p % kPreDepth], ring[(p + kPreDepth - 1) % kPreDepth], rb, voff, w,
                lane, acc);
  }
}

// The streaming kernel on prepacked B: A goes through the same LDS ring of
// pairs (its scale pieces share the copy with B's prepacked scale block), B
// through a ring of kPreDepth pairs in each wave's registers.  The per-wave
// k-step split, the MFMA order and the reduction are those of
// gemm_stream_kernel, so both give bit-identical fp32 sums.
//
// K runs in straight-line chunks of 8, 4 and 1 pairs (K = 4096 is one chunk);
// both rings refill at each chunk boundary.
template <class C>
__global__ __launch_bounds__(kThreads) void gemm_stream_pre_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  static_assert(C::PRE, "prepacked-B configuration");
  static_assert(kPreDepth >= C::NP, "B runs at least as far ahead as A");
  static_assert((C::NP - 1) * C::PAIR_LOADS + (kPreDepth - 1) * kPreBLoads <= 63, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t MXFP4_LDS* lds = (uint8_t MXFP4_LDS*)smem;
  int tm, tn;
  if (!stream_coords(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
  // Wave-uniform values go to scalar registers, so the buffer resource below is
  // provably uniform (no per-lane loop around each load) and the loop control
  // stays scalar.
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int m0 = tm * C::BM, n0 = tn * kBN;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

  v16f acc[C::MB][2];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int np = __builtin_amdgcn_readfirstlane(args.k / 512);
  PreCopies<C> src;
  make_pre_copies<C>(src, args, m0, tn, np, w, lane);
  // this panel's prepacked codes: np blocks of 16 KB (32 * k <= 2^29 bytes)
  const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(args.b_q + (int64_t)tn * np * kPreCodeBlock,
                                                 (uint32_t)np * kPreCodeBlock);
  const uint32_t voff = w * 4096 + lane * 16;

  int p0 = 0;
  for (; p0 + 8 <= np; p0 += 8) pre_chunk<C, 8>(lds, src, p0, rb, voff, w, lane, acc);
  if (p0 + 4 <= np) {
    pre_chunk<C, 4>(lds, src, p0, rb, voff, w, lane, acc);
    p0 += 4;
  }
  for (; p0 < np; ++p0) pre_chunk<C, 1>(lds, src, p0, rb, voff, w, lane, acc);

  MXFP4_WAIT_VMCNT(0);
  __syncthreads();   // every wave is done with the ring

  stream_epilogue<C>(acc, args, m0, n0, lds, w, lane);
}

template <class C>
hipError_t launch_pre_cfg(const GemmArgs& args, hipStream_t stream) {
  const auto kernel = gemm_stream_pre_kernel<C>;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  const int tiles_n = (args.n + kBN - 1) / kBN;
  const int tiles_m = (args.m + C::BM - 1) / C::BM;
  const int64_t blocks = (int64_t)tiles_m * ((tiles_n + 7) / 8) * 8;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), C::LDS, stream, args, tiles_m, tiles_n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Both operands prepacked.  The prepacked layout is defined for any [rows, K]
// MXFP4 operand (64-row panels, 512-K pairs), so A can take it too.  Then each
// wave loads its A and B operands straight into registers, 1 KB contiguous per
// load, and the main loop touches no LDS: no copies into LDS, no barriers and
// no hand-counted waits (the compiler's waits on the loaded registers are
// exact, every vector-memory op being a plain load).  The per-wave k-step
// split, the MFMA order and the fixed-order reduction are those of
// gemm_stream_kernel, so the results are bit-identical to it.
//
// Row tiles: BM = 32 * MB rows of A.  MB = 4 and 2 cover whole 64-row A
// panels (two and one); MB = 1 covers half a panel (j_a = tile % 2).
//
// A8 (W4A8): A in the FP8 prepacked layout (include/mxfp8.h): per pair, wave
// and u = 2s + j, two 1 KB pieces holding each lane's first and last 16 codes
// (32 KB per panel and pair instead of 16 KB); the scale bytes as for MXFP4.
// The per-wave k-step split, the MFMA order and the reduction are those of
// the W4A8 prepacked-weight streaming kernel, so the results are bit-identical
// to it.
template <int MB, bool A8>
struct PPPair {
  typename std::conditional<A8, v8i, v4i>::type a[MB][2];   // [row block][stage]
  v4i b[4];       // [2s + j]
  int sa[MB > 1 ? MB / 2 : 1];   // one scale word per A panel
  int sb;
};

constexpr int kPPDepth = 4;    // pairs in each wave's register ring
constexpr int kPPDepth8 = 2;   // the same with FP8 A (twice the A registers per pair)
constexpr int kPre8CodeBlock = 32 * 1024;   // FP8 A codes per 64-row panel and 512-K pair

template <int MB, bool A8>
__device__ __forceinline__ void pp_load(PPPair<MB, A8>& r, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rsa,
                                        __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rsb, uint32_t qoff,
                                        uint32_t aoff, uint32_t soff, uint32_t a_panel_q, uint32_t a_panel_s, int ja,
                                        int p) {
  // Every offset is in the per-lane offset, which the buffer range check
  // covers: a pair past the last reads zeros without touching memory.  The
  // scheduling barriers keep each pair's loads together where they are
  // written: without them the scheduler pulls every MFMA up next to the loads
  // it consumes, the registers are then reused pair after pair, and each load
  // waits for the MFMAs of the pair before it (no prefetch at all).
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t pq = qoff + (uint32_t)p * kPreCodeBlock, ps = soff + (uint32_t)p * kPreScaleBlock;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    r.b[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb, pq + u * 1024, 0, kLoadNT));
  r.sb = (int)__builtin_amdgcn_raw_buffer_load_b32(rsb, ps, 0, kLoadNT);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int panel = MB > 1 ? i / 2 : 0;
    const int j = MB > 1 ? (i & 1) : ja;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (A8) {
        const uint32_t pa = aoff + (uint32_t)p * kPre8CodeBlock + panel * a_panel_q + (2 * s + j) * 2048;
        const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, pa, 0, 0));
        const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, pa + 1024, 0, 0));
        r.a[i][s] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      } else {
        r.a[i][s] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, pq + panel * a_panel_q + (2 * s + j) * 1024, 0, 0));
      }
    }
  }
#pragma unroll
  for (int pn = 0; pn < (MB > 1 ? MB / 2 : 1); ++pn)
    r.sa[pn] = (int)__builtin_amdgcn_raw_buffer_load_b32(rsa, ps + pn * a_panel_s, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// One MFMA of the pair: B column block (op_sel OB of sb) times A row block
// (op_sel OA of sa), FP4 x FP4 or FP4 x FP8.
template <bool A8, int OB, int OA, class AV>
__device__ __forceinline__ v16f pp_mfma(v4i b, AV a, v16f acc, int sb, int sa) {
  if constexpr (A8)
    return mfma32_fp4_fp8_sel<OB, OA>(b, a, acc, sb, sa);
  else
    return mfma32_fp4_sel<OB, OA>(b, a, acc, sb, sa);
}

template <int MB, int S, bool A8>
__device__ __forceinline__ void pp_mma_stage(const PPPair<MB, A8>& r, int ja, v16f (&acc)[MB][2]) {
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if constexpr (MB > 1) {
      const int sa = r.sa[i / 2];
      if (i & 1) {
        acc[i][0] = pp_mfma<A8, 2 * S, 2 * S + 1>(r.b[2 * S], r.a[i][S], acc[i][0], r.sb, sa);
        acc[i][1] = pp_mfma<A8, 2 * S + 1, 2 * S + 1>(r.b[2 * S + 1], r.a[i][S], acc[i][1], r.sb, sa);
      } else {
        acc[i][0] = pp_mfma<A8, 2 * S, 2 * S>(r.b[2 * S], r.a[i][S], acc[i][0], r.sb, sa);
        acc[i][1] = pp_mfma<A8, 2 * S + 1, 2 * S>(r.b[2 * S + 1], r.a[i][S], acc[i][1], r.sb, sa);
      }
    } else {
      const int sa = r.sa[0] >> (8 * ja);   // byte 2s + ja moved to byte 2s
      acc[i][0] = pp_mfma<A8, 2 * S, 2 * S>(r.b[2 * S], r.a[i][S], acc[i][0], r.sb, sa);
      acc[i][1] = pp_mfma<A8, 2 * S + 1, 2 * S>(r.b[2 * S + 1], r.a[i][S], acc[i][1], r.sb, sa);
    }
  }
}

// Stage 0 then stage 1, row blocks in order: the streaming kernel's order.
template <int MB, bool A8>
__device__ __forceinline__ void pp_mma(const PPPair<MB, A8>& r, int ja, v16f (&acc)[MB][2]) {
  pp_mma_stage<MB, 0, A8>(r, ja, acc);
  pp_mma_stage<MB, 1, A8>(r, ja, acc);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pp_rsrc(const uint8_t* base, int64_t bytes) {
  return uniform_rsrc(base, (uint32_t)bytes);
}

// CH pairs starting at pair p0 as straight-line code: a ring of kPPDepth
// pairs, loads for pair p + kPPDepth - 1 issued before the MFMAs of pair p.
// The ring lives only inside one chunk, so no register crosses a loop
// back-edge (a ring carried round a loop made the compiler copy and spill it).
template <int MB, int CH, bool A8>
__device__ __forceinline__ void pp_chunk(int p0, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rsa,
                                         __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rsb, uint32_t qoff,
                                         uint32_t aoff, uint32_t soff, uint32_t a_panel_q, uint32_t panel_s, int ja,
                                         v16f (&acc)[MB][2]) {
  constexpr int D = A8 ? kPPDepth8 : kPPDepth;
  PPPair<MB, A8> ring[D];
#pragma unroll
  for (int q = 0; q < D - 1; ++q)
    if (q < CH) pp_load<MB, A8>(ring[q], ra, rsa, rb, rsb, qoff, aoff, soff, a_panel_q, panel_s, ja, p0 + q);
#pragma unroll
  for (int p = 0; p < CH; ++p) {
    if (p + D - 1 < CH)
      pp_load<MB, A8>(ring[(p + D - 1) % D], ra, rsa, rb, rsb, qoff, aoff, soff, a_panel_q, panel_s, ja,
                      p0 + p + D - 1);
    pp_mma<MB, A8>(ring[p % D], ja, acc);
  }
}

// Split-K of the both-prepacked kernel, for shapes with fewer output tiles
// than compute units (the decode down projection: 64 column panels).  Each
// output tile's K is cut into `splits` ranges of `pairs_per_split` 512-K pairs
// (the last may be shorter), one workgroup each.  A workgroup writes its
// reduced fp32 tile to the workspace and bumps the tile's arrival counter; the
// last to arrive sums the partial tiles in split order 0, 1, ... (so results
// do not depend on timing), stores C and returns the counter to zero.
//
// Visibility across workgroups, which may run on different XCDs with separate
// L2 caches: the partial tiles are written and read with device-coherent
// accesses (the sc1 cache policy, the one relaxed device-scope atomic loads
// and stores compile to), and every writer waits for its stores to complete
// before its arrival.  Only these lines bypass the L2; the device-scope
// release / acquire fences would instead write back and invalidate the whole
// L2, which made the older split-K kernel many times slower.
struct PPSplit {
  int splits;            // K ranges per output tile
  int pairs_per_split;   // 512-K pairs per range
  int* counters;         // [tiles], zero between launches
  float* partials;       // [tiles][splits][units][64 lanes][4 floats]
};

constexpr int kCoherent = 16;   // buffer cache policy bits: sc1 (device-coherent)

// This workgroup's part of the split-K reduction of output tile `tile`: own[]
// holds the wave's summed units of K range `split`.  Returns false for every
// workgroup but the last to arrive; that one gets the sum over all ranges in
// own[].
template <class C>
__device__ __forceinline__ bool combine_splits(v4f (&own)[C::MB * 2], const PPSplit& sk, int tile, int split,
                                               uint8_t MXFP4_LDS* lds, int w, int lane) {
  constexpr int U = C::MB * 8, UW = U / 4;
  const __amdgpu_buffer_rsrc_t rp = uniform_rsrc((const uint8_t*)(sk.partials + (int64_t)tile * sk.splits * U * 256),
                                                 (uint32_t)(sk.splits * U * 1024));
#pragma unroll
  for (int t = 0; t < UW; ++t)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, own[t]), rp,
                                           (uint32_t)(((split * U + w * UW + t) * 64 + lane) * 16), 0, kCoherent);
  MXFP4_WAIT_VMCNT(0);   // this thread's partial stores have completed
  __syncthreads();
  // the reduction exchange area is free again: its first word carries the verdict
  int MXFP4_LDS* last = (int MXFP4_LDS*)lds;
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(&sk.counters[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = prev == sk.splits - 1;
    if (prev == sk.splits - 1) __hip_atomic_store(&sk.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*last) return false;
  // The other ranges' partial tiles in groups of four: a group's loads are all
  // issued before any is used (one memory round trip per group; loaded one at
  // a time the sum took longer than the whole main loop), then added in range
  // order, this workgroup's own range (already in registers) taking its place
  // in that order.  The loads are unconditional (past the last range they
  // reread it) so that no branch makes the compiler wait between them.
  constexpr int G = 4;
  const int others = sk.splits - 1;
  v4f sum[UW];
  bool own_done = false;
  const auto add = [&](int sp, const v4f (&v)[UW]) {
#pragma unroll
    for (int t = 0; t < UW; ++t) sum[t] = sp == 0 ? v[t] : sum[t] + v[t];
  };
  for (int o0 = 0; o0 < others; o0 += G) {
    v4f part[G][UW];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int o = min(o0 + g, others - 1);
      const int sp = o < split ? o : o + 1;
#pragma unroll
      for (int t = 0; t < UW; ++t)
        part[g][t] = __builtin_bit_cast(
            v4f, __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(((sp * U + w * UW + t) * 64 + lane) * 16), 0,
                                                       kCoherent));
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the group before the first add
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int o = o0 + g;
      if (o >= others) break;
      const int sp = o < split ? o : o + 1;
      if (!own_done && sp > split) {
        add(split, own);
        own_done = true;
      }
      add(sp, part[g]);
    }
  }
  if (!own_done) add(split, own);
#pragma unroll
  for (int t = 0; t < UW; ++t) own[t] = sum[t];
  return true;
}

// K in chunks of 8 pairs (K = 4096 is one chunk), then one of 4, then single
// pairs; the pipeline refills at each chunk boundary.  SPLIT: the workgroup
// covers one K range of its tile (combine_splits).
template <int MB, bool SPLIT, bool A8 = false>
__global__ __launch_bounds__(kThreads) void gemm_pp_kernel(GemmArgs args, int tiles_m, int tiles_n, PPSplit sk) {
  using EC = StreamCfg<MB, 2, false, true>;   // epilogue layout (reduction area and C tile)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t MXFP4_LDS* lds = (uint8_t MXFP4_LDS*)smem;
  const int splits = SPLIT ? sk.splits : 1;
  int tm, tv;
  if (!stream_coords(blockIdx.x, tiles_m, tiles_n * splits, tm, tv)) return;
  tm = __builtin_amdgcn_readfirstlane(tm);
  tv = __builtin_amdgcn_readfirstlane(tv);
  const int tn = tv / splits, split = tv - tn * splits;
  const int m0 = tm * EC::BM, n0 = tn * kBN;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int np = __builtin_amdgcn_readfirstlane(args.k / 512);
  const int p_begin = SPLIT ? split * sk.pairs_per_split : 0;
  const int p_end = SPLIT ? min(np, p_begin + sk.pairs_per_split) : np;

  // B: this column panel.  A: the tile's row panels (MB = 1: half of one);
  // the A panels that exist for this tile (the last tile of a ragged m may
  // have fewer): loads past them fall outside the resource and read zeros.
  const int64_t panel_q = (int64_t)np * kPreCodeBlock, panel_s = (int64_t)np * kPreScaleBlock;
  const int64_t a_panel_q = (int64_t)np * (A8 ? kPre8CodeBlock : kPreCodeBlock);
  const int a_panel0 = m0 / 64;
  const int a_panels = min(MB > 1 ? MB / 2 : 1, (args.m + 63) / 64 - a_panel0);
  const int ja = MB > 1 ? 0 : (tm & 1);
  const __amdgpu_buffer_rsrc_t rb = pp_rsrc(args.b_q + tn * panel_q, panel_q);
  const __amdgpu_buffer_rsrc_t rsb = pp_rsrc(args.b_s + tn * panel_s, panel_s);
  const __amdgpu_buffer_rsrc_t ra = pp_rsrc(args.a_q + a_panel0 * a_panel_q, a_panels * a_panel_q);
  const __amdgpu_buffer_rsrc_t rsa = pp_rsrc(args.a_s + a_panel0 * panel_s, a_panels * panel_s);
  const uint32_t qoff = w * 4096 + lane * 16, soff = w * 256 + lane * 4;
  const uint32_t aoff = A8 ? w * 8192 + lane * 16 : qoff;   // FP8 A: 8 KB per wave and pair

  v16f acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const uint32_t apq = (uint32_t)a_panel_q, ps = (uint32_t)panel_s;
  int p0 = p_begin;
  for (; p0 + 8 <= p_end; p0 += 8) pp_chunk<MB, 8, A8>(p0, ra, rsa, rb, rsb, qoff, aoff, soff, apq, ps, ja, acc);
  if (p0 + 4 <= p_end) {
    pp_chunk<MB, 4, A8>(p0, ra, rsa, rb, rsb, qoff, aoff, soff, apq, ps, ja, acc);
    p0 += 4;
  }
  for (; p0 < p_end; ++p0) pp_chunk<MB, 1, A8>(p0, ra, rsa, rb, rsb, qoff, aoff, soff, apq, ps, ja, acc);

  v4f own[MB * 2];
  reduce_units<EC>(acc, lds, w, lane, own);
  if constexpr (SPLIT) {
    if (!combine_splits<EC>(own, sk, tm * tiles_n + tn, split, lds, w, lane)) return;
  }
  store_units<EC>(own, args, m0, n0, lds, w, lane);
}

template <int MB>
int pp_tiles(const GemmArgs& args) {
  return ((args.m + 32 * MB - 1) / (32 * MB)) * ((args.n + kBN - 1) / kBN);
}

template <int MB, bool SPLIT, bool A8 = false>
hipError_t launch_pp_cfg(const GemmArgs& args, const PPSplit& sk, hipStream_t stream) {
  using EC = StreamCfg<MB, 2, false, true>;
  constexpr int lds_bytes = EC::XCH + EC::C_TILE;
  const auto kernel = gemm_pp_kernel<MB, SPLIT, A8>;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  const int tiles_n = (args.n + kBN - 1) / kBN;
  const int tiles_m = (args.m + EC::BM - 1) / EC::BM;
  const int64_t virt_n = (int64_t)tiles_n * (SPLIT ? sk.splits : 1);
  const int64_t blocks = (int64_t)tiles_m * ((virt_n + 7) / 8) * 8;
  if (virt_n > 0x7FFFFFFF || !grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), lds_bytes, stream, args, tiles_m, tiles_n, sk);
  return hipGetLastError();
}

// Pairs per K range for a request of `splits` ranges over np pairs:
// ceil(np / splits), rounded up to a multiple of 4 when above 4, so that a
// range runs as whole 8- and 4-pair chunks (single pairs run with no loads in
// flight behind them: 7-pair ranges measured about twice as slow per pair).
int pp_range_pairs(int np, int splits) {
  int pps = (np + splits - 1) / splits;
  if (pps > 4) pps = (pps + 3) & ~3;
  return pps;
}

template <int MB>
hipError_t launch_pp(const GemmArgs& args, int splits, void* workspace, hipStream_t stream) {
  PPSplit sk{1, args.k / 512, nullptr, nullptr};
  if (splits <= 1) return launch_pp_cfg<MB, false>(args, sk, stream);
  const int np = args.k / 512;
  sk.pairs_per_split = pp_range_pairs(np, splits);
  sk.splits = (np + sk.pairs_per_split - 1) / sk.pairs_per_split;   // no empty range
  if (sk.splits <= 1) return launch_pp_cfg<MB, false>(args, sk, stream);
  if (pp_tiles<MB>(args) > kPPMaxTiles) return hipErrorInvalidValue;
  sk.counters = (int*)workspace;
  sk.partials = (float*)((uint8_t*)workspace + kPPCounterBytes);
  return launch_pp_cfg<MB, true>(args, sk, stream);
}

}  // namespace

bool stream_supported(const GemmArgs& args) {
  return args.k % 512 == 0 && ((reinterpret_cast<uintptr_t>(args.a_s) | reinterpret_cast<uintptr_t>(args.b_s)) & 15) == 0;
}

hipError_t launch_gemm_stream(const GemmArgs& args, hipStream_t stream) {
  if (args.m <= 0 || args.n <= 0) return hipSuccess;
  if (!stream_supported(args)) return hipErrorInvalidValue;
  if (args.m <= 32) return launch_cfg<StreamCfg<1, 5>>(args, stream);
  if (args.m <= 64) return launch_cfg<StreamCfg<2, 4>>(args, stream);
  return launch_cfg<StreamCfg<4, 3>>(args, stream);
}

hipError_t launch_gemm_w4a8_stream(const GemmArgs& args, hipStream_t stream) {
  if (args.m <= 0 || args.n <= 0) return hipSuccess;
  if (!stream_supported(args)) return hipErrorInvalidValue;
  if (args.m <= 32) return launch_cfg<StreamCfg<1, 4, true>>(args, stream);
  return launch_cfg<StreamCfg<2, 3, true>>(args, stream);
}

void prepacked_sizes(int64_t n, int64_t k, int64_t* code_bytes, int64_t* scale_bytes) {
  const int64_t panels = (n + kBN - 1) / kBN;
  *code_bytes = panels * kBN * (k / 2);
  *scale_bytes = panels * kBN * (k / 32);
}

hipError_t launch_prepack_weight(const uint8_t* b_q, const uint8_t* b_s, int n, int k, uint8_t* bp_q, uint8_t* bp_s,
                                 hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (k <= 0 || k % 512) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)((n + kBN - 1) / kBN) * (k / 512);
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, b_q, b_s, n, k, bp_q, bp_s);
  return hipGetLastError();
}

hipError_t launch_gemm_stream_prepacked(const GemmArgs& args, hipStream_t stream) {
  if (args.m <= 0 || args.n <= 0) return hipSuccess;
  if (!stream_supported(args)) return hipErrorInvalidValue;
  using Pre1 = StreamCfg<1, 4, false, true>;
  using Pre2 = StreamCfg<2, 4, false, true>;
  using Pre4 = StreamCfg<4, 4, false, true>;
  if (args.m <= 32) return launch_pre_cfg<Pre1>(args, stream);
  if (args.m <= 64) return launch_pre_cfg<Pre2>(args, stream);
  return launch_pre_cfg<Pre4>(args, stream);
}

// Row blocks per tile of the both-prepacked kernel for m rows.
static int pp_mb(int m) { return m <= 32 ? 1 : (m <= 64 ? 2 : 4); }

int pp_effective_splits(int k, int splits) {
  const int np = k / 512;
  if (splits <= 1 || np <= 1) return 1;
  const int pps = pp_range_pairs(np, splits);
  return (np + pps - 1) / pps;
}

int pp_auto_splits(int m, int n, int k, int num_cus) {
  const int mb = pp_mb(m);
  const int64_t tiles = (int64_t)((m + 32 * mb - 1) / (32 * mb)) * ((n + kBN - 1) / kBN);
  const int np = k / 512;
  // enough K ranges to give most compute units a workgroup, each at least
  // two pairs long, and at most 16
  int s = (int)std::min<int64_t>(16, std::max<int64_t>(1, num_cus / std::max<int64_t>(1, tiles)));
  s = std::min(s, std::max(1, np / 2));
  if (tiles > kPPMaxTiles) s = 1;
  return pp_effective_splits(k, s);
}

size_t pp_workspace_bytes(int m, int n, int k, int splits) {
  const int s = pp_effective_splits(k, splits);
  if (s <= 1) return 0;
  const int mb = pp_mb(m);
  const int64_t tiles = (int64_t)((m + 32 * mb - 1) / (32 * mb)) * ((n + kBN - 1) / kBN);
  if (tiles > kPPMaxTiles) return 0;
  return kPPCounterBytes + (size_t)tiles * s * (32 * mb) * kBN * sizeof(float);
}

hipError_t launch_gemm_w4a8_stream_prepacked(const GemmArgs& args, hipStream_t stream) {
  if (args.m <= 0 || args.n <= 0) return hipSuccess;
  if (!stream_supported(args)) return hipErrorInvalidValue;
  // FP8 A rows are twice as long: a 128-row tile fits two pairs of A in LDS
  using Pre1 = StreamCfg<1, 4, true, true>;
  using Pre2 = StreamCfg<2, 4, true, true>;
  using Pre4 = StreamCfg<4, 2, true, true>;
  if (args.m <= 32) return launch_pre_cfg<Pre1>(args, stream);
  if (args.m <= 64) return launch_pre_cfg<Pre2>(args, stream);
  return launch_pre_cfg<Pre4>(args, stream);
}

hipError_t launch_gemm_w4a8_both_prepacked(const GemmArgs& args, hipStream_t stream) {
  if (args.m <= 0 || args.n <= 0) return hipSuccess;
  if (args.k <= 0 || args.k % 512) return hipErrorInvalidValue;
  const PPSplit sk{1, args.k / 512, nullptr, nullptr};
  if (args.m <= 32) return launch_pp_cfg<1, false, true>(args, sk, stream);
  if (args.m <= 64) return launch_pp_cfg<2, false, true>(args, sk, stream);
  return launch_pp_cfg<4, false, true>(args, sk, stream);
}

hipError_t launch_gemm_both_prepacked(const GemmArgs& args, int splits, void* workspace, hipStream_t stream) {
  if (args.m <= 0 || args.n <= 0) return hipSuccess;
  if (args.k <= 0 || args.k % 512) return hipErrorInvalidValue;
  if (args.m <= 32) return launch_pp<1>(args, splits, workspace, stream);
  if (args.m <= 64) return launch_pp<2>(args, splits, workspace, stream);
  return launch_pp<4>(args, splits, workspace, stream);
}

}  // namespace mxfp4
