// Measurement probes for the ceilings the GEMM kernels are compared against
// (declared in include/mxfp4_probe.h): the scaled-MFMA rate of a kernel that
// does nothing else (FP4 x FP4, or FP4 x FP8 as in the W4A8 GEMM), and the
// read rate of a plain streaming kernel.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kMfmaProbeThreads = 512;   // 8 waves per workgroup, 2 per SIMD
constexpr int kReadProbeThreads = 256;

// One wave: a 4 x 2 grid of 32x32 accumulator blocks fed by four A and two B
// operand registers, the MFMA pattern of one k-step of a tile-kernel wave.
// After every k-step the operands are rotated and mixed (VALU work that
// overlaps the matrix core), so consecutive MFMAs see new data.  With A8 the A
// operands are FP8 (32 bytes per lane; the upper half is derived from the
// seed's next row) with every NaN pattern masked off (exponent bit 0 cleared).
template <bool A8>
__global__ __launch_bounds__(kMfmaProbeThreads) void mfma_probe_kernel(const v4i* seed, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  constexpr int kNoNaN = (int)0xF7F7F7F7u;
  v4i a[4], b[2];
  v4i a_hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = seed[i * 64 + lane];
    a_hi[i] = seed[((i + 1) & 3) * 64 + lane] ^ (v4i){0x1b873593, 0x6b43a9b5, 0x3c6ef372, 0x0f1bbcdc};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = seed[(4 + j) * 64 + lane];
  const int scale = 0x7f7f7f7f;   // E8M0 byte 127 (2^0) in every byte
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (A8) {
          const v8i a8 = {a[i].x & kNoNaN, a[i].y & kNoNaN, a[i].z & kNoNaN, a[i].w & kNoNaN,
                          a_hi[i].x & kNoNaN, a_hi[i].y & kNoNaN, a_hi[i].z & kNoNaN, a_hi[i].w & kNoNaN};
          acc[i][j] = mfma32_fp4_fp8<0>(b[j], a8, acc[i][j], scale, scale);
        } else {
          acc[i][j] = mfma32_fp4<0>(b[j], a[i], acc[i][j], scale, scale);
        }
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (v4i){a[i].y, a[i].z, a[i].w, a[i].x ^ 0x5bd1e995};
    if constexpr (A8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a_hi[i] = (v4i){a_hi[i].w ^ 0x2545f491, a_hi[i].x, a_hi[i].y, a_hi[i].z};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = (v4i){b[j].w, b[j].x ^ 0x27d4eb2f, b[j].y, b[j].z};
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[(int64_t)blockIdx.x * kMfmaProbeThreads + threadIdx.x] = s;
}

// Grid-stride streaming read with 16 independent 16-byte loads in flight per
// thread per round; loads past the end are predicated off, so the last round
// overlaps too.  (Measured earlier: one 256-thread workgroup per CU with 16
// loads in flight read fastest, 6.1-6.5 TB/s over large buffers.)
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(kReadProbeThreads) void read_probe_kernel(const v4i* src, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * kReadProbeThreads;
  v4i x = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * kReadProbeThreads + threadIdx.x; i < n16; i += kReadUnroll * stride) {
    v4i v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < n16 ? src[j] : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u];
  }
  out[(int64_t)blockIdx.x * kReadProbeThreads + threadIdx.x] = (uint32_t)(x.x ^ x.y ^ x.z ^ x.w);
}

}  // namespace

double probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * (kMfmaProbeThreads / 64) * iters * 8 * (2.0 * 32 * 32 * 64);
}

hipError_t launch_probe_mfma(const void* seed, void* out, int blocks, int iters, bool a_fp8, hipStream_t stream) {
  if (!grid_fits(blocks, kMfmaProbeThreads)) return hipErrorInvalidConfiguration;
  if (a_fp8)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3((unsigned)blocks), dim3(kMfmaProbeThreads), 0, stream,
                       (const v4i*)seed, (float*)out, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3((unsigned)blocks), dim3(kMfmaProbeThreads), 0, stream,
                       (const v4i*)seed, (float*)out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t bytes, void* out, int blocks, hipStream_t stream) {
  if (!grid_fits(blocks, kReadProbeThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kReadProbeThreads), 0, stream,
                     (const v4i*)src, bytes / 16, (uint32_t*)out);
  return hipGetLastError();
}

}  // namespace mxfp4
