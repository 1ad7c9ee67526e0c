// Bandwidth path of the block-scaled FP4 GEMM for small M (decode), gfx950.
//
// At decode (M <= 128) the GEMM is bound by streaming the packed weight B once
// from HBM (the quadbit README, "Real Llama-3-8B GEMM shapes": decode is
// memory-bound, and small shapes leave too few output tiles to fill the chip;
// its serving section splits K over more CTAs with an fp32 reduction to fill
// the machine).  Here:
//  * a workgroup owns all M rows (up to 128) and BN = 64 (or 32) output
//    columns; with splits == 1 (the automatic choice) it covers the whole K, so
//    no partial sums leave the workgroup;
//  * its 4 waves split K into quarters.  Each wave streams its A and B
//    fragments straight from global memory into MFMA operand registers (no LDS
//    round trip: every byte is used by exactly one wave), in chunks of 128 K
//    held in a 3-deep register ring, so up to three chunks are in flight while
//    the MFMAs of the oldest run (fully unrolled for the common chunk counts);
//  * the four wave accumulators are summed through LDS in a fixed order;
//  * with splits > 1 (only when asked for) each workgroup covers a K-range,
//    writes its fp32 partial tile to the workspace and bumps a per-column-tile
//    counter; the last of the `splits` workgroups to arrive sums the partials
//    in split order (deterministic), writes C and resets the counter to zero.
//    The counters live in the first 64 KiB of the workspace for every shape;
//    the partial tiles follow.  Cross-workgroup visibility needs agent-scope
//    release/acquire, which on this chip writes back and invalidates L2, so
//    this mode is slow and is never chosen automatically.
// MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 with the B fragment as first operand,
// so each lane ends up with runs of 4 consecutive output columns.  Within a
// 128-K chunk, k-step s (0..1) reads 32-blocks 2s (lanes 0..31) and 2s+1
// (lanes 32..63); a row's 4 scale bytes for the chunk arrive as one 32-bit load.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 128;      // K elements per pipeline step (2 MFMA k-steps)
constexpr int kMaxM = 128;
// The counters occupy a fixed region at the start of every workspace, whatever
// the shape, so a workspace reused across shapes keeps them at zero.
constexpr size_t kSplitkCounterBytes = 65536;

template <int MB, int NI>
struct Chunk {
  v4i a[MB][2];     // [m-block][k-step]
  v4i b[NI][2];
  int as[MB];       // the row's 4 scale bytes of this chunk
  int bs[NI];
};

// Loads one 128-element K chunk.  FULL: k % 128 == 0, every chunk lies inside
// K and each row's 4 scale bytes are one aligned 32-bit load; otherwise scales
// are read byte by byte and 32-blocks past K get zero codes.
template <int MB, int NI, bool FULL>
__device__ __forceinline__ void load_chunk(Chunk<MB, NI>& f, const GemmArgs& args, int n0, int chunk, int lane) {
  const int64_t kb = args.k / 2, ks = args.k / 32;
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int kblocks = args.k / 32;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = min(32 * i + r32, args.m - 1);
    const uint8_t* ap = args.a_q + row * kb + chunk * 64 + half * 16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (FULL || chunk * 4 + 2 * s + half < kblocks) f.a[i][s] = *(const v4i*)(ap + 32 * s);
      else f.a[i][s] = v4i{0, 0, 0, 0};
    }
    const uint8_t* sp = args.a_s + row * ks + chunk * 4;
    if (FULL) {
      f.as[i] = *(const int*)sp;
    } else {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (chunk * 4 + b < kblocks ? (uint32_t)sp[b] : 127u) << (8 * b);
      f.as[i] = (int)w;
    }
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int row = min(n0 + 32 * j + r32, args.n - 1);
    const uint8_t* bp = args.b_q + row * kb + chunk * 64 + half * 16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (FULL || chunk * 4 + 2 * s + half < kblocks) f.b[j][s] = *(const v4i*)(bp + 32 * s);
      else f.b[j][s] = v4i{0, 0, 0, 0};
    }
    const uint8_t* sp = args.b_s + row * ks + chunk * 4;
    if (FULL) {
      f.bs[j] = *(const int*)sp;
    } else {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (chunk * 4 + b < kblocks ? (uint32_t)sp[b] : 127u) << (8 * b);
      f.bs[j] = (int)w;
    }
  }
}

// Lanes 32..63 feed the odd 32-block of each k-step: their scale word moves
// right by one byte, so k-step s takes byte 2s.
template <int MB, int NI>
__device__ __forceinline__ void mma_chunk(const Chunk<MB, NI>& f, v16f (&acc)[MB][NI], int shift) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int sa = (int)((uint32_t)f.as[i] >> shift);
        const int sb = (int)((uint32_t)f.bs[j] >> shift);
        if (s == 0) acc[i][j] = mfma32_fp4<0>(f.b[j][0], f.a[i][0], acc[i][j], sb, sa);
        else acc[i][j] = mfma32_fp4<2>(f.b[j][1], f.a[i][1], acc[i][j], sb, sa);
      }
}

__device__ __forceinline__ void chunk_range(int nchunks, int parts, int idx, int& lo, int& hi) {
  lo = (int)((int64_t)nchunks * idx / parts);
  hi = (int)((int64_t)nchunks * (idx + 1) / parts);
}

// A wave's NCH chunks, fully unrolled over a 3-deep register ring: chunk c+3
// is requested as soon as chunk c's MFMAs are issued, so up to three chunks are
// in flight.  Straight-line code lets the compiler place exact vmcnt waits.
// `rot` rotates the chunk order (see the kernel); chunk indices wrap at nchunks.
template <int MB, int NI, int NCH>
__device__ __forceinline__ void wave_mainloop_fixed(v16f (&acc)[MB][NI], const GemmArgs& args, int n0, int lo,
                                                    int rot, int nchunks, int lane) {
  const int shift = 8 * (lane >> 5);
  auto at = [&](int c) { const int x = lo + c + rot; return x >= nchunks ? x - nchunks : x; };
  Chunk<MB, NI> ring[3];
#pragma unroll
  for (int c = 0; c < (NCH < 3 ? NCH : 3); ++c) load_chunk<MB, NI, true>(ring[c], args, n0, at(c), lane);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    mma_chunk<MB, NI>(ring[c % 3], acc, shift);
    if (c + 3 < NCH) load_chunk<MB, NI, true>(ring[c % 3], args, n0, at(c + 3), lane);
  }
}

// Any chunk count: two register buffers in a rolled loop.
template <int MB, int NI, bool FULL>
__device__ __forceinline__ void wave_mainloop(v16f (&acc)[MB][NI], const GemmArgs& args, int n0, int lo,
                                              int hi, int lane) {
  const int shift = 8 * (lane >> 5);
  Chunk<MB, NI> b0, b1;
  int c = lo;
  if (c < hi) load_chunk<MB, NI, FULL>(b0, args, n0, c, lane);
  if (c + 1 < hi) load_chunk<MB, NI, FULL>(b1, args, n0, c + 1, lane);
  for (; c + 1 < hi; c += 2) {
    mma_chunk<MB, NI>(b0, acc, shift);
    if (c + 2 < hi) load_chunk<MB, NI, FULL>(b0, args, n0, c + 2, lane);
    mma_chunk<MB, NI>(b1, acc, shift);
    if (c + 3 < hi) load_chunk<MB, NI, FULL>(b1, args, n0, c + 3, lane);
  }
  if (c < hi) mma_chunk<MB, NI>(b0, acc, shift);
}

template <int MB, int NI>
__global__ __launch_bounds__(kThreads) void gemm_splitk_kernel(GemmArgs args, int tiles_n, int splits,
                                                               float* __restrict__ partials,
                                                               int* __restrict__ counters) {
  constexpr int BN = 32 * NI;
  constexpr int TM = 32 * MB;            // rows held per tile
  constexpr int TILE = TM * BN;          // fp32 elements per tile
  __shared__ float red[4 * TILE];
  __shared__ int last_flag;

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tn = blockIdx.x % tiles_n;
  const int split = blockIdx.x / tiles_n;
  const int n0 = tn * BN;

  const int nchunks = (args.k + kChunk - 1) / kChunk;
  int wlo, whi;
  {
    int slo, shi;
    chunk_range(nchunks, splits, split, slo, shi);
    int a, b;
    chunk_range(shi - slo, 4, w, a, b);
    wlo = slo + a;
    whi = slo + b;
  }

  v16f acc[MB][NI];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Every workgroup reads all of A.  Were they all to walk K in the same order,
  // every CU would ask for the same A lines at the same moment and queue on
  // one L2 channel; with splits == 1 each workgroup instead starts its K walk
  // at its own offset (A is small enough to stay resident in L2).  Only when
  // the four waves' ranges are equal: then they all take the same loop, and a
  // rotation that only some of them applied would cover chunks twice or not
  // at all.
  const int rot = (splits == 1 && nchunks % 4 == 0) ? (int)(((int64_t)tn * 7) % nchunks) : 0;
  if (args.k % kChunk == 0 && (splits == 1 || rot == 0)) {
    switch (whi - wlo) {   // wave-uniform
      case 8: wave_mainloop_fixed<MB, NI, 8>(acc, args, n0, wlo, rot, nchunks, lane); break;
      case 16: wave_mainloop_fixed<MB, NI, 16>(acc, args, n0, wlo, rot, nchunks, lane); break;
      case 28: wave_mainloop_fixed<MB, NI, 28>(acc, args, n0, wlo, rot, nchunks, lane); break;
      case 4: wave_mainloop_fixed<MB, NI, 4>(acc, args, n0, wlo, rot, nchunks, lane); break;
      default: wave_mainloop<MB, NI, true>(acc, args, n0, wlo, whi, lane); break;
    }
  } else {
    wave_mainloop<MB, NI, false>(acc, args, n0, wlo, whi, lane);
  }

  // each wave stores its accumulators as a row-major [TM][BN] fp32 tile
  float* mine = red + w * TILE;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * i + (lane & 31);
        const int col = 32 * j + 8 * q + 4 * (lane >> 5);
        *(float4*)(mine + r * BN + col) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  __syncthreads();

  // fixed-order sum of the 4 wave partials; thread t owns float4 slots t, t+256, ...
  constexpr int SLOTS = TILE / 4;
  constexpr int PER_THREAD = (SLOTS + kThreads - 1) / kThreads;
  float4 sum[PER_THREAD];
#pragma unroll
  for (int u = 0; u < PER_THREAD; ++u) {
    const int e = (threadIdx.x + u * kThreads) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e < TILE) {
      s = *(const float4*)(red + e);
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        const float4 o = *(const float4*)(red + ww * TILE + e);
        s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
      }
    }
    sum[u] = s;
  }

  const int m = args.m, n = args.n;
  const bool vec_ok = (n & 3) == 0;
  auto store = [&](int e, float4 s) {
    const int r = e / BN, col = n0 + (e % BN);
    if (e >= TILE || r >= m) return;
    const int64_t off = (int64_t)r * n + col;
    if (args.c_f32) {
      float* cp = (float*)args.c + off;
      if (vec_ok && col + 3 < n) { *(float4*)cp = s; return; }
      if (col + 0 < n) cp[0] = s.x;
      if (col + 1 < n) cp[1] = s.y;
      if (col + 2 < n) cp[2] = s.z;
      if (col + 3 < n) cp[3] = s.w;
    } else {
      uint16_t* cp = (uint16_t*)args.c + off;
      if (vec_ok && col + 3 < n) { *(uint2*)cp = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)); return; }
      if (col + 0 < n) cp[0] = (uint16_t)f32_to_bf16_bits(s.x);
      if (col + 1 < n) cp[1] = (uint16_t)f32_to_bf16_bits(s.y);
      if (col + 2 < n) cp[2] = (uint16_t)f32_to_bf16_bits(s.z);
      if (col + 3 < n) cp[3] = (uint16_t)f32_to_bf16_bits(s.w);
    }
  };

  if (splits == 1) {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) store((threadIdx.x + u * kThreads) * 4, sum[u]);
    return;
  }

  // publish this split's partial tile: partials[tile][split][TILE]
  float* my_part = partials + ((int64_t)tn * splits + split) * TILE;
#pragma unroll
  for (int u = 0; u < PER_THREAD; ++u) {
    const int e = (threadIdx.x + u * kThreads) * 4;
    if (e < TILE) *(float4*)(my_part + e) = sum[u];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(&counters[tn], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == splits - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* parts = partials + (int64_t)tn * splits * TILE;
#pragma unroll
  for (int u = 0; u < PER_THREAD; ++u) {
    const int e = (threadIdx.x + u * kThreads) * 4;
    if (e >= TILE) continue;
    float4 s = *(const float4*)(parts + e);
    for (int sp = 1; sp < splits; ++sp) {
      const float4 o = *(const float4*)(parts + (int64_t)sp * TILE + e);
      s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
    }
    store(e, s);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&counters[tn], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int mblocks_for(int m) { return m <= 32 ? 1 : (m <= 64 ? 2 : 4); }

// 64 output columns per workgroup when that still gives most CUs a workgroup,
// 32 otherwise (each workgroup reads all of A, so wider tiles read A fewer times).
int nblocks_for(int n, int num_cus) { return (n + 63) / 64 >= (num_cus * 3) / 4 ? 2 : 1; }

}  // namespace

namespace {
__global__ __launch_bounds__(kThreads) void clear_counters_kernel(int* counters, int n) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) counters[i] = 0;
}
}  // namespace

hipError_t launch_splitk_clear_counters(void* workspace, hipStream_t stream) {
  const int n = splitk_max_tiles();
  hipLaunchKernelGGL(clear_counters_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                     (int*)workspace, n);
  return hipGetLastError();
}

size_t splitk_workspace_bytes(int m, int n, int k, int splits) {
  (void)k;
  if (splits <= 1) return 0;
  // partial tiles of the narrower (32-column) tiling, which needs the most room
  const size_t per_split = (size_t)((n + 31) / 32) * 32 * (32 * mblocks_for(m)) * sizeof(float);
  return kSplitkCounterBytes + per_split * splits;
}

int splitk_max_tiles() { return (int)(kSplitkCounterBytes / sizeof(int)); }

int splitk_auto_splits(int m, int n, int k, int num_cus) {
  (void)m; (void)n; (void)k; (void)num_cus;
  return 1;   // full-K workgroups: no partial sums cross workgroups (see the file comment)
}

hipError_t launch_gemm_splitk(const GemmArgs& args, int splits, void* workspace, hipStream_t stream,
                              int num_cus) {
  if (args.m > kMaxM) return hipErrorInvalidValue;
  const int ni = nblocks_for(args.n, num_cus);
  const int bn = 32 * ni;
  const int tiles_n = (args.n + bn - 1) / bn;
  int* counters = nullptr;
  float* partials = nullptr;
  if (splits > 1) {
    if (tiles_n > splitk_max_tiles()) return hipErrorInvalidValue;
    counters = (int*)workspace;
    partials = (float*)((char*)workspace + kSplitkCounterBytes);
  }
  const int64_t blocks = (int64_t)tiles_n * splits;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  const int mb = mblocks_for(args.m);
#define MXFP4_LAUNCH(MB_, NI_)                                                                               \
  hipLaunchKernelGGL((gemm_splitk_kernel<MB_, NI_>), grid, dim3(kThreads), 0, stream, args, tiles_n, splits, \
                     partials, counters)
  if (ni == 2) {
    if (mb == 1) MXFP4_LAUNCH(1, 2);
    else if (mb == 2) MXFP4_LAUNCH(2, 2);
    else MXFP4_LAUNCH(4, 2);
  } else {
    if (mb == 1) MXFP4_LAUNCH(1, 1);
    else if (mb == 2) MXFP4_LAUNCH(2, 1);
    else MXFP4_LAUNCH(4, 1);
  }
#undef MXFP4_LAUNCH
  return hipGetLastError();
}

}  // namespace mxfp4
