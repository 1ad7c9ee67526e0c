// Bandwidth path of the block-scaled FP4 GEMM for small M (decode), gfx950.
//
// At decode (M <= 128) the GEMM is bound by streaming the packed weight B once
// from HBM (the quadbit README, "Real Llama-3-8B GEMM shapes": decode is
// memory-bound, and small shapes leave too few output tiles to fill the chip;
// its serving section splits K over more CTAs with an fp32 reduction to fill
// the machine).  Here:
//  * a workgroup owns all M rows (up to 128) and 64 output columns, and a
//    K-range given by `splits` (K is cut into 128-element chunks);
//  * inside the workgroup the 4 waves split that K-range again, each streaming
//    its own B rows straight from global memory into MFMA operand registers
//    (no LDS round trip: every B byte is used by exactly one wave), with the
//    next chunk's loads issued before the current chunk's MFMAs;
//  * A (small, shared by every workgroup) is read through L2 the same way;
//  * the four wave accumulators are summed through LDS in a fixed order;
//  * with splits > 1 each workgroup writes its fp32 partial tile to the
//    workspace and bumps a per-column-tile counter; the last of the `splits`
//    workgroups to arrive sums all partials in split order (deterministic),
//    writes C and resets the counter to zero for the next call.  The counters
//    live in the first 64 KiB of the workspace for every shape (so reuse across
//    shapes never finds partial sums where a counter should be) and the
//    partial tiles follow.
// MFMA use is as in the tile kernels: v_mfma_scale_f32_32x32x64_f8f6f4 with
// the B fragment as first operand, so each lane ends up with 4-column runs.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;          // output columns per workgroup
constexpr int kNI = kBN / 32;    // 32-column MFMA blocks per wave
constexpr int kChunk = 128;      // K elements per pipeline step (2 MFMA k-steps)

template <int MB>
struct Frag {
  v4i a[MB][2];     // [m-block][k-step]
  v4i b[kNI][2];
  int as[MB];       // scale words, already shifted for this lane's K-half
  int bs[kNI];
};

// Loads one 128-element K chunk. FULL: k % 128 == 0, so every chunk lies inside
// K and each row's scale word is an aligned 32-bit load; otherwise scales are
// read byte by byte and 32-blocks past K get zero codes.
template <int MB, bool FULL>
__device__ __forceinline__ void load_chunk(Frag<MB>& f, const GemmArgs& args, int n0, int chunk, int lane) {
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
    uint32_t w;
    if (FULL) {
      w = *(const uint32_t*)sp;
    } else {
      w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (chunk * 4 + b < kblocks ? (uint32_t)sp[b] : 127u) << (8 * b);
    }
    f.as[i] = (int)(w >> (8 * half));
  }
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    const int row = min(n0 + 32 * j + r32, args.n - 1);
    const uint8_t* bp = args.b_q + row * kb + chunk * 64 + half * 16;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (FULL || chunk * 4 + 2 * s + half < kblocks) f.b[j][s] = *(const v4i*)(bp + 32 * s);
      else f.b[j][s] = v4i{0, 0, 0, 0};
    }
    const uint8_t* sp = args.b_s + row * ks + chunk * 4;
    uint32_t w;
    if (FULL) {
      w = *(const uint32_t*)sp;
    } else {
      w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (chunk * 4 + b < kblocks ? (uint32_t)sp[b] : 127u) << (8 * b);
    }
    f.bs[j] = (int)(w >> (8 * half));
  }
}

template <int MB>
__device__ __forceinline__ void mma_chunk(const Frag<MB>& f, v16f (&acc)[MB][kNI]) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) {
      acc[i][j] = mfma32_fp4<0>(f.b[j][0], f.a[i][0], acc[i][j], f.bs[j], f.as[i]);
      acc[i][j] = mfma32_fp4<2>(f.b[j][1], f.a[i][1], acc[i][j], f.bs[j], f.as[i]);
    }
}

__device__ __forceinline__ void chunk_range(int nchunks, int parts, int idx, int& lo, int& hi) {
  lo = (int)((int64_t)nchunks * idx / parts);
  hi = (int)((int64_t)nchunks * (idx + 1) / parts);
}

template <int MB>
__global__ __launch_bounds__(kThreads) void gemm_splitk_kernel(GemmArgs args, int tiles_n, int splits,
                                                               float* __restrict__ partials,
                                                               int* __restrict__ counters) {
  constexpr int TM = 32 * MB;            // rows held per tile
  constexpr int TILE = TM * kBN;         // fp32 elements per tile
  __shared__ float red[4 * TILE];
  __shared__ int last_flag;

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tn = blockIdx.x % tiles_n;
  const int split = blockIdx.x / tiles_n;
  const int n0 = tn * kBN;

  const int nchunks = (args.k + kChunk - 1) / kChunk;
  const bool aligned = (args.k % kChunk) == 0;
  int wlo, whi;
  {
    int slo, shi;
    chunk_range(nchunks, splits, split, slo, shi);
    int a, b;
    chunk_range(shi - slo, 4, w, a, b);
    wlo = slo + a;
    whi = slo + b;
  }

  v16f acc[MB][kNI];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  if (wlo < whi) {
    Frag<MB> cur, nxt;
    if (aligned) load_chunk<MB, true>(cur, args, n0, wlo, lane);
    else load_chunk<MB, false>(cur, args, n0, wlo, lane);
    for (int c = wlo; c < whi; ++c) {
      if (c + 1 < whi) {
        if (aligned) load_chunk<MB, true>(nxt, args, n0, c + 1, lane);
        else load_chunk<MB, false>(nxt, args, n0, c + 1, lane);
      }
      mma_chunk<MB>(cur, acc);
      cur = nxt;
    }
  }

  // each wave stores its accumulators as a row-major [TM][kBN] fp32 tile
  float* mine = red + w * TILE;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * i + (lane & 31);
        const int col = 32 * j + 8 * q + 4 * (lane >> 5);
        *(float4*)(mine + r * kBN + col) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  __syncthreads();

  // fixed-order sum of the 4 wave partials; thread t owns float4 slots t, t+256, ...
  constexpr int SLOTS = TILE / 4;
  float4 sum[SLOTS / kThreads];
#pragma unroll
  for (int u = 0; u < SLOTS / kThreads; ++u) {
    const int e = (threadIdx.x + u * kThreads) * 4;
    float4 s = *(const float4*)(red + e);
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      const float4 o = *(const float4*)(red + ww * TILE + e);
      s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
    }
    sum[u] = s;
  }

  const int m = args.m, n = args.n;
  const bool vec_ok = (n & 3) == 0;
  auto store = [&](int e, float4 s) {
    const int r = e / kBN, col = n0 + (e % kBN);
    if (r >= m) return;
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
    for (int u = 0; u < SLOTS / kThreads; ++u) store((threadIdx.x + u * kThreads) * 4, sum[u]);
    return;
  }

  // publish this split's partial tile: partials[tile][split][TILE]
  float* my_part = partials + ((int64_t)tn * splits + split) * TILE;
#pragma unroll
  for (int u = 0; u < SLOTS / kThreads; ++u) *(float4*)(my_part + (threadIdx.x + u * kThreads) * 4) = sum[u];
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
  for (int u = 0; u < SLOTS / kThreads; ++u) {
    const int e = (threadIdx.x + u * kThreads) * 4;
    float4 s = *(const float4*)(parts + e);
    for (int sp = 1; sp < splits; ++sp) {
      const float4 o = *(const float4*)(parts + (int64_t)sp * TILE + e);
      s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
    }
    store(e, s);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&counters[tn], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kMaxM = 128;
// The counters occupy a fixed region at the start of every workspace, whatever
// the shape, so a workspace reused across shapes keeps them at zero.
constexpr size_t kSplitkCounterBytes = 65536;

int mblocks_for(int m) { return m <= 32 ? 1 : (m <= 64 ? 2 : 4); }

}  // namespace

size_t splitk_workspace_bytes(int m, int n, int k, int splits) {
  (void)k;
  if (splits <= 1) return 0;
  const int tiles_n = (n + kBN - 1) / kBN;
  const size_t tile = (size_t)32 * mblocks_for(m) * kBN;
  const size_t part = (size_t)tiles_n * splits * tile * sizeof(float);
  return kSplitkCounterBytes + part;
}

int splitk_max_tiles() { return (int)(kSplitkCounterBytes / sizeof(int)); }

int splitk_auto_splits(int m, int n, int k, int num_cus) {
  (void)m;
  const int tiles_n = (n + kBN - 1) / kBN;
  const int nchunks = (k + kChunk - 1) / kChunk;
  // enough workgroups to cover every CU, each wave keeping >= 2 chunks of work
  int s = 1;
  if (tiles_n > splitk_max_tiles()) return 1;
  while (tiles_n * s < num_cus && nchunks / (4 * (s * 2)) >= 2 && s < 64) s *= 2;
  return s;
}

hipError_t launch_gemm_splitk(const GemmArgs& args, int splits, void* workspace, hipStream_t stream) {
  if (args.m > kMaxM) return hipErrorInvalidValue;
  const int tiles_n = (args.n + kBN - 1) / kBN;
  int* counters = nullptr;
  float* partials = nullptr;
  if (splits > 1) {
    if (tiles_n > splitk_max_tiles()) return hipErrorInvalidValue;
    counters = (int*)workspace;
    partials = (float*)((char*)workspace + kSplitkCounterBytes);
  }
  const dim3 grid((unsigned)(tiles_n * splits));
  switch (mblocks_for(args.m)) {
    case 1: hipLaunchKernelGGL((gemm_splitk_kernel<1>), grid, dim3(kThreads), 0, stream, args, tiles_n, splits, partials, counters); break;
    case 2: hipLaunchKernelGGL((gemm_splitk_kernel<2>), grid, dim3(kThreads), 0, stream, args, tiles_n, splits, partials, counters); break;
    default: hipLaunchKernelGGL((gemm_splitk_kernel<4>), grid, dim3(kThreads), 0, stream, args, tiles_n, splits, partials, counters); break;
  }
  return hipGetLastError();
}

}  // namespace mxfp4
