// Measurement probes for the ceilings the GEMM kernels are compared against
// (declared in include/mxfp4_probe.h): the FP4 scaled-MFMA rate of a kernel
// that does nothing else, and the read rate of a plain streaming kernel.
#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

constexpr int kMfmaProbeThreads = 512;   // 8 waves per workgroup, 2 per SIMD
constexpr int kReadProbeThreads = 256;

// One wave: a 4 x 2 grid of 32x32 accumulator blocks fed by four A and two B
// operand registers, the MFMA pattern of one k-step of a tile-kernel wave.
// After every k-step the operands are rotated and mixed (VALU work that
// overlaps the matrix core), so consecutive MFMAs see new data.
__global__ __launch_bounds__(kMfmaProbeThreads) void mfma_probe_kernel(const v4i* seed, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  v4i a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = seed[i * 64 + lane];
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
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32_fp4<0>(b[j], a[i], acc[i][j], scale, scale);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (v4i){a[i].y, a[i].z, a[i].w, a[i].x ^ 0x5bd1e995};
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

hipError_t launch_probe_mfma(const void* seed, void* out, int blocks, int iters, hipStream_t stream) {
  if (!grid_fits(blocks, kMfmaProbeThreads)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kMfmaProbeThreads), 0, stream,
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
