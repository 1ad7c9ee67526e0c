// C ABI of the MXFP4 library: argument checks, per-shape kernel choice, launches.
// Entry points and their contracts are documented in include/mxfp4.h, include/mxfp8.h,
// include/mxfp4_moe.h, include/mxfp4_producers.h and include/nvfp4.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/mxfp4.h"
#include "../../include/mxfp4_probe.h"
#include "../../include/mxfp8.h"
#include "../../include/mxfp4_moe.h"
#include "../../include/mxfp4_producers.h"
#include "../../include/nvfp4.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

mxfp4_status_t fail(mxfp4_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

struct DeviceInfo {
  bool valid = false;
  bool gfx950 = false;
  int num_cus = 0;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mutex;

mxfp4_status_t current_device(DeviceInfo& out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MXFP4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MXFP4_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_devices_mutex);
  DeviceInfo& d = g_devices[dev];
  if (!d.valid) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MXFP4_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.valid = true;
  }
  out = d;
  if (!out.gfx950) return fail(MXFP4_ERR_UNSUPPORTED, "the current device is not gfx950");
  return MXFP4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;   // m, n: keeps row and tile indices in int32 range
constexpr int32_t kMaxPPSplits = 16;             // K ranges of the both-prepacked split-K GEMM
// k: the tile kernels address a tile's operand rows with 32-bit byte offsets
// from the tile's first row, (row in tile) * k/2 with up to 256 rows.
constexpr int64_t kMaxK = (int64_t)1 << 24;

mxfp4_status_t check_k(int64_t k) {
  if (k <= 0 || k % 32 != 0) return fail(MXFP4_ERR_INVALID_ARG, "k must be a positive multiple of 32 (got %lld)", (long long)k);
  if (k > kMaxK) return fail(MXFP4_ERR_INVALID_ARG, "k too large (%lld > %lld)", (long long)k, (long long)kMaxK);
  return MXFP4_OK;
}

mxfp4_status_t check_ptr(const void* p, const char* name, unsigned align = 16) {
  if (!p) return fail(MXFP4_ERR_INVALID_ARG, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0)
    return fail(MXFP4_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, align);
  return MXFP4_OK;
}

// Scale arrays are read as 32-bit words (four 32-blocks) when k % 128 == 0 and
// byte by byte otherwise.
unsigned scale_align(int64_t k) { return k % 128 == 0 ? 4u : 1u; }

mxfp4_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MXFP4_OK;
}

#define MXFP4_TRY(expr)                 \
  do {                                  \
    mxfp4_status_t s_ = (expr);         \
    if (s_ != MXFP4_OK) return s_;      \
  } while (0)

struct Choice {
  mxfp4_kernel_t kernel;
  int splits;
};

// Per-shape kernel choice (`stream_ok`: the streaming kernel's k and scale
// alignment requirements hold).
Choice choose(int64_t m, int64_t n, int64_t k, int num_cus, bool stream_ok) {
  if (m <= 128) {
    if (stream_ok) return {MXFP4_KERNEL_STREAM, 0};
    return {MXFP4_KERNEL_SPLITK, mxfp4::splitk_auto_splits((int)m, (int)n, (int)k, num_cus)};
  }
  const int64_t tiles256 = ((m + 255) / 256) * ((n + 255) / 256);
  if (tiles256 >= num_cus) return {MXFP4_KERNEL_TILE256, 0};
  return {MXFP4_KERNEL_TILE128, 0};
}

mxfp4_status_t resolve(int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel, int32_t splits,
                       int num_cus, bool stream_ok, Choice& out) {
  switch (kernel) {
    case MXFP4_KERNEL_AUTO: out = choose(m, n, k, num_cus, stream_ok); return MXFP4_OK;
    case MXFP4_KERNEL_TILE256:
    case MXFP4_KERNEL_TILE128: out = {kernel, 0}; return MXFP4_OK;
    case MXFP4_KERNEL_PERSISTENT:
      if (!stream_ok || k % 1024 != 0)
        return fail(MXFP4_ERR_INVALID_ARG,
                    "the persistent kernel needs k %% 1024 == 0 and 16-byte aligned scale arrays");
      out = {kernel, 0};
      return MXFP4_OK;
    case MXFP4_KERNEL_STREAM:
      if (!stream_ok)
        return fail(MXFP4_ERR_INVALID_ARG, "the stream kernel needs k %% 512 == 0 and 16-byte aligned scale arrays");
      out = {kernel, 0};
      return MXFP4_OK;
    case MXFP4_KERNEL_SPLITK:
      if (m > 128) return fail(MXFP4_ERR_INVALID_ARG, "the split-K kernel takes m <= 128 (got %lld)", (long long)m);
      if (splits < 0 || splits > 64) return fail(MXFP4_ERR_INVALID_ARG, "splits must be 0..64 (got %d)", splits);
      out = {kernel, splits == 0 ? mxfp4::splitk_auto_splits((int)m, (int)n, (int)k, num_cus) : splits};
      if (out.splits > 1 && (n + 63) / 64 > mxfp4::splitk_max_tiles())
        return fail(MXFP4_ERR_INVALID_ARG, "split-K with splits > 1 supports n <= %d", 64 * mxfp4::splitk_max_tiles());
      return MXFP4_OK;
  }
  return fail(MXFP4_ERR_INVALID_ARG, "unknown kernel id %d", (int)kernel);
}

size_t workspace_for(const Choice& c, int64_t m, int64_t n, int64_t k) {
  if (c.kernel == MXFP4_KERNEL_SPLITK) return mxfp4::splitk_workspace_bytes((int)m, (int)n, (int)k, c.splits);
  return 0;
}

int query_num_cus() {
  DeviceInfo d;
  if (current_device(d) != MXFP4_OK) return 256;
  return d.num_cus;
}

mxfp4_status_t check_gemm_args(const void* a_q, const void* a_s, const void* b_q, const void* b_s,
                               const void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (m > kMaxDim || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "m or n too large");
  MXFP4_TRY(check_k(k));
  if (c_type != MXFP4_OUT_BF16 && c_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)c_type);
  if (m > 0) {
    MXFP4_TRY(check_ptr(a_q, "a_q"));
    MXFP4_TRY(check_ptr(a_s, "a_s", scale_align(k)));
  }
  if (n > 0) {
    MXFP4_TRY(check_ptr(b_q, "b_q"));
    MXFP4_TRY(check_ptr(b_s, "b_s", scale_align(k)));
  }
  if (m > 0 && n > 0) MXFP4_TRY(check_ptr(c, "c"));
  return MXFP4_OK;
}

}  // namespace

extern "C" {

int mxfp4_abi_version(void) { return MXFP4_ABI_VERSION; }

const char* mxfp4_status_string(mxfp4_status_t s) {
  switch (s) {
    case MXFP4_OK: return "ok";
    case MXFP4_ERR_INVALID_ARG: return "invalid argument";
    case MXFP4_ERR_UNSUPPORTED: return "unsupported device";
    case MXFP4_ERR_WORKSPACE: return "workspace too small";
    case MXFP4_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mxfp4_last_error(void) { return g_last_error; }

mxfp4_status_t mxfp4_quantize(const void* x_bf16, int64_t rows, int64_t k, void* q, void* scales,
                              void* stream) {
  if (rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative rows");
  MXFP4_TRY(check_k(k));
  if (rows > ((int64_t)1 << 40) / k) return fail(MXFP4_ERR_INVALID_ARG, "rows * k too large");
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(q, "q", 4));
  MXFP4_TRY(check_ptr(scales, "scales", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_quantize(x_bf16, rows, k, q, scales, (hipStream_t)stream, dev.num_cus),
                    "quantize launch");
}

mxfp4_status_t mxfp8_quantize(const void* x_bf16, int64_t rows, int64_t k, void* q8, void* scales, void* stream) {
  if (rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative rows");
  MXFP4_TRY(check_k(k));
  if (rows > ((int64_t)1 << 40) / k) return fail(MXFP4_ERR_INVALID_ARG, "rows * k too large");
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(q8, "q8", 8));
  MXFP4_TRY(check_ptr(scales, "scales", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_quantize_mxfp8(x_bf16, rows, k, q8, scales, (hipStream_t)stream, dev.num_cus),
                    "mxfp8 quantize launch");
}

size_t mxfp4_gemm_nt_ex_workspace_size(int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel, int32_t splits) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 32 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxK) return 0;
  // without the pointers the alignment is unknown: size for the non-streaming choice
  Choice c;
  if (resolve(m, n, k, kernel, splits, query_num_cus(), (kernel == MXFP4_KERNEL_STREAM || kernel == MXFP4_KERNEL_PERSISTENT) && k % 512 == 0, c) != MXFP4_OK)
    return 0;
  return workspace_for(c, m, n, k);
}

size_t mxfp4_gemm_nt_workspace_size(int64_t m, int64_t n, int64_t k) {
  return mxfp4_gemm_nt_ex_workspace_size(m, n, k, MXFP4_KERNEL_AUTO, 0);
}

}  // extern "C"

namespace {

// The no-allocation variant's scratch: a file-scope device array (one copy on
// each GPU the library runs on, held until the process ends).  Host code uses
// only the per-device address hipGetSymbolAddress returns for it, never the
// array's name.
constexpr size_t kNoAllocScratchBytes = MXFP4_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device, looked up once per device
// with that device current.
mxfp4_status_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MXFP4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MXFP4_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MXFP4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MXFP4_OK;
}

// mxfp4_gemm_nt_ex's body; with `noalloc`, the workspace is the library's
// scratch array (workspace arguments ignored).
mxfp4_status_t gemm_nt_ex_impl(const void* a_q, const void* a_s, const void* b_q, const void* b_s, void* c,
                               mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel,
                               int32_t splits, void* workspace, size_t workspace_bytes, void* stream,
                               bool noalloc) {
  MXFP4_TRY(check_gemm_args(a_q, a_s, b_q, b_s, c, c_type, m, n, k));
  if (kernel < MXFP4_KERNEL_AUTO || kernel > MXFP4_KERNEL_PERSISTENT)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown kernel id %d", (int)kernel);
  if (m == 0 || n == 0) return MXFP4_OK;
  const bool stream_ok = k % 512 == 0 && ((reinterpret_cast<uintptr_t>(a_s) | reinterpret_cast<uintptr_t>(b_s)) & 15) == 0;
  Choice ch;
  // the forced stream and persistent kernels' requirements need no device
  if (kernel == MXFP4_KERNEL_STREAM || kernel == MXFP4_KERNEL_PERSISTENT)
    MXFP4_TRY(resolve(m, n, k, kernel, splits, 0, stream_ok, ch));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  MXFP4_TRY(resolve(m, n, k, kernel, splits, dev.num_cus, stream_ok, ch));
  const size_t need = workspace_for(ch, m, n, k);
  if (noalloc) {
    if (need > kNoAllocScratchBytes)
      return fail(MXFP4_ERR_WORKSPACE, "the no-allocation entry point's scratch holds %zu bytes; this call needs %zu",
                  kNoAllocScratchBytes, need);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      MXFP4_TRY(device_scratch(&workspace));
      workspace_bytes = kNoAllocScratchBytes;
      // the array keeps the last call's contents: zero the arrival counters first
      MXFP4_TRY(hip_status(mxfp4::launch_splitk_clear_counters(workspace, (hipStream_t)stream),
                           "scratch counter clear launch"));
    }
  } else if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(MXFP4_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(MXFP4_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  }
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  hipError_t e;
  switch (ch.kernel) {
    case MXFP4_KERNEL_SPLITK:
      e = mxfp4::launch_gemm_splitk(args, ch.splits, workspace, (hipStream_t)stream, dev.num_cus);
      break;
    case MXFP4_KERNEL_STREAM: e = mxfp4::launch_gemm_stream(args, (hipStream_t)stream); break;
    case MXFP4_KERNEL_TILE128: e = mxfp4::launch_gemm_tile(args, mxfp4::kTile128, (hipStream_t)stream); break;
    case MXFP4_KERNEL_PERSISTENT:
      e = mxfp4::launch_gemm_tile_persistent(args, dev.num_cus, 0, (hipStream_t)stream);
      break;
    default: e = mxfp4::launch_gemm_tile(args, mxfp4::kTile256, (hipStream_t)stream); break;
  }
  return hip_status(e, "gemm launch");
}

}  // namespace

extern "C" {

mxfp4_status_t mxfp4_gemm_nt_ex(const void* a_q, const void* a_s, const void* b_q, const void* b_s,
                                void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                                mxfp4_kernel_t kernel, int32_t splits, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return gemm_nt_ex_impl(a_q, a_s, b_q, b_s, c, c_type, m, n, k, kernel, splits, workspace, workspace_bytes,
                         stream, false);
}

mxfp4_status_t mxfp4_gemm_nt_ex_noalloc(const void* a_q, const void* a_s, const void* b_q, const void* b_s,
                                        void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                                        mxfp4_kernel_t kernel, int32_t splits, void* stream) {
  return gemm_nt_ex_impl(a_q, a_s, b_q, b_s, c, c_type, m, n, k, kernel, splits, nullptr, 0, stream, true);
}

mxfp4_status_t mxfp4_gemm_nt(const void* a_q, const void* a_s, const void* b_q, const void* b_s, void* c,
                             mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return mxfp4_gemm_nt_ex(a_q, a_s, b_q, b_s, c, c_type, m, n, k, MXFP4_KERNEL_AUTO, 0, workspace,
                          workspace_bytes, stream);
}

mxfp4_status_t mxfp4_prepacked_weight_size(int64_t n, int64_t k, int64_t* code_bytes, int64_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return fail(MXFP4_ERR_INVALID_ARG, "size outputs are NULL");
  if (n < 0 || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "n out of range");
  MXFP4_TRY(check_k(k));
  if (k % 512) return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  mxfp4::prepacked_sizes(n, k, code_bytes, scale_bytes);
  return MXFP4_OK;
}

mxfp4_status_t mxfp4_prepack_weight(const void* b_q, const void* b_s, int64_t n, int64_t k, void* bp_q, void* bp_s,
                                    void* stream) {
  int64_t cb, sb;
  MXFP4_TRY(mxfp4_prepacked_weight_size(n, k, &cb, &sb));
  if (n == 0) return MXFP4_OK;
  if ((n + 63) / 64 * (k / 512) > (int64_t)0xFFFFFFFF / 256) return fail(MXFP4_ERR_INVALID_ARG, "weight too large");
  MXFP4_TRY(check_ptr(b_q, "b_q"));
  MXFP4_TRY(check_ptr(b_s, "b_s", 1));
  MXFP4_TRY(check_ptr(bp_q, "bp_q"));
  MXFP4_TRY(check_ptr(bp_s, "bp_s"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_prepack_weight((const uint8_t*)b_q, (const uint8_t*)b_s, (int)n, (int)k,
                                                 (uint8_t*)bp_q, (uint8_t*)bp_s, (hipStream_t)stream),
                    "prepack launch");
}

mxfp4_status_t mxfp4_gemm_nt_prepacked(const void* a_q, const void* a_s, const void* bp_q, const void* bp_s, void* c,
                                       mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream) {
  if (m < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (m > kMaxDim || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "m or n too large");
  MXFP4_TRY(check_k(k));
  if (k % 512) return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (c_type != MXFP4_OUT_BF16 && c_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)c_type);
  if (m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(a_q, "a_q"));
  MXFP4_TRY(check_ptr(a_s, "a_s"));
  MXFP4_TRY(check_ptr(bp_q, "bp_q"));
  MXFP4_TRY(check_ptr(bp_s, "bp_s"));
  MXFP4_TRY(check_ptr(c, "c"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)bp_q;
  args.b_s = (const uint8_t*)bp_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  return hip_status(mxfp4::launch_gemm_stream_prepacked(args, (hipStream_t)stream), "prepacked gemm launch");
}

mxfp4_status_t mxfp8_gemm_w4a8_nt_prepacked(const void* a_q8, const void* a_s, const void* bp_q, const void* bp_s,
                                            void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                                            void* stream) {
  if (m < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (m > kMaxDim || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "m or n too large");
  MXFP4_TRY(check_k(k));
  if (k % 512) return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (c_type != MXFP4_OUT_BF16 && c_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)c_type);
  if (m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(a_q8, "a_q8"));
  MXFP4_TRY(check_ptr(a_s, "a_s"));
  MXFP4_TRY(check_ptr(bp_q, "bp_q"));
  MXFP4_TRY(check_ptr(bp_s, "bp_s"));
  MXFP4_TRY(check_ptr(c, "c"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q8;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)bp_q;
  args.b_s = (const uint8_t*)bp_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  return hip_status(mxfp4::launch_gemm_w4a8_stream_prepacked(args, (hipStream_t)stream),
                    "prepacked w4a8 gemm launch");
}

mxfp4_status_t mxfp8_quantize_prepacked(const void* x_bf16, int64_t rows, int64_t k, void* ap_q8, void* ap_s,
                                        void* stream) {
  int64_t cb, sb;
  MXFP4_TRY(mxfp4_prepacked_weight_size(rows, k, &cb, &sb));
  if (rows == 0) return MXFP4_OK;
  if ((rows + 63) / 64 * 64 > ((int64_t)1 << 40) / k) return fail(MXFP4_ERR_INVALID_ARG, "rows * k too large");
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(ap_q8, "ap_q8"));
  MXFP4_TRY(check_ptr(ap_s, "ap_s", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_quantize_mxfp8_prepacked(x_bf16, rows, k, ap_q8, ap_s, (hipStream_t)stream,
                                                           dev.num_cus), "mxfp8 prepacked quantize launch");
}

mxfp4_status_t mxfp8_gemm_w4a8_nt_prepacked_ab(const void* ap_q8, const void* ap_s, const void* bp_q,
                                               const void* bp_s, void* c, mxfp4_out_t c_type, int64_t m, int64_t n,
                                               int64_t k, void* stream) {
  if (m < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (m > kMaxDim || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "m or n too large");
  MXFP4_TRY(check_k(k));
  if (k % 512) return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (c_type != MXFP4_OUT_BF16 && c_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)c_type);
  if (m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(ap_q8, "ap_q8"));
  MXFP4_TRY(check_ptr(ap_s, "ap_s"));
  MXFP4_TRY(check_ptr(bp_q, "bp_q"));
  MXFP4_TRY(check_ptr(bp_s, "bp_s"));
  MXFP4_TRY(check_ptr(c, "c"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)ap_q8;
  args.a_s = (const uint8_t*)ap_s;
  args.b_q = (const uint8_t*)bp_q;
  args.b_s = (const uint8_t*)bp_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  return hip_status(mxfp4::launch_gemm_w4a8_both_prepacked(args, (hipStream_t)stream),
                    "both-prepacked w4a8 gemm launch");
}

mxfp4_status_t mxfp4_quantize_prepacked(const void* x_bf16, int64_t rows, int64_t k, void* ap_q, void* ap_s,
                                        void* stream) {
  int64_t cb, sb;
  MXFP4_TRY(mxfp4_prepacked_weight_size(rows, k, &cb, &sb));
  if (rows == 0) return MXFP4_OK;
  if ((rows + 63) / 64 * 64 > ((int64_t)1 << 40) / k) return fail(MXFP4_ERR_INVALID_ARG, "rows * k too large");
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(ap_q, "ap_q"));
  MXFP4_TRY(check_ptr(ap_s, "ap_s", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_quantize_prepacked(x_bf16, rows, k, ap_q, ap_s, (hipStream_t)stream, dev.num_cus),
                    "prepacked quantize launch");
}

size_t mxfp4_gemm_nt_prepacked_ab_workspace_size(int64_t m, int64_t n, int64_t k, int32_t splits) {
  if (m <= 0 || n <= 0 || m > kMaxDim || n > kMaxDim || check_k(k) != MXFP4_OK || k % 512) return 0;
  if (splits < 0 || splits > kMaxPPSplits) return 0;
  const int s = splits == 0 ? mxfp4::pp_auto_splits((int)m, (int)n, (int)k, query_num_cus()) : splits;
  return mxfp4::pp_workspace_bytes((int)m, (int)n, (int)k, s);
}

mxfp4_status_t mxfp4_gemm_nt_prepacked_ab_ex(const void* ap_q, const void* ap_s, const void* bp_q, const void* bp_s,
                                             void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                                             int32_t splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (m > kMaxDim || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "m or n too large");
  MXFP4_TRY(check_k(k));
  if (k % 512) return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (c_type != MXFP4_OUT_BF16 && c_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)c_type);
  if (splits < 0 || splits > kMaxPPSplits)
    return fail(MXFP4_ERR_INVALID_ARG, "splits must be 0..%d (got %d)", kMaxPPSplits, splits);
  if (m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(ap_q, "ap_q"));
  MXFP4_TRY(check_ptr(ap_s, "ap_s"));
  MXFP4_TRY(check_ptr(bp_q, "bp_q"));
  MXFP4_TRY(check_ptr(bp_s, "bp_s"));
  MXFP4_TRY(check_ptr(c, "c"));
  // an explicit split of a shape with too many output tiles is refused before any device call
  if (splits > 1 && mxfp4::pp_effective_splits((int)k, splits) > 1 &&
      mxfp4::pp_workspace_bytes((int)m, (int)n, (int)k, splits) == 0)
    return fail(MXFP4_ERR_INVALID_ARG, "split-K supports at most 16384 output tiles (64-column panels x row tiles)");
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  const int s = splits == 0 ? mxfp4::pp_auto_splits((int)m, (int)n, (int)k, dev.num_cus) : splits;
  const size_t need = mxfp4::pp_workspace_bytes((int)m, (int)n, (int)k, s);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(MXFP4_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(MXFP4_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  }
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)ap_q;
  args.a_s = (const uint8_t*)ap_s;
  args.b_q = (const uint8_t*)bp_q;
  args.b_s = (const uint8_t*)bp_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  return hip_status(mxfp4::launch_gemm_both_prepacked(args, need > 0 ? s : 1, workspace, (hipStream_t)stream),
                    "prepacked gemm launch");
}

mxfp4_status_t mxfp4_gemm_nt_prepacked_ab(const void* ap_q, const void* ap_s, const void* bp_q, const void* bp_s,
                                          void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream) {
  return mxfp4_gemm_nt_prepacked_ab_ex(ap_q, ap_s, bp_q, bp_s, c, c_type, m, n, k, 1, nullptr, 0, stream);
}

size_t mxfp4_grouped_gemm_nt_workspace_size(int64_t total_m, int32_t num_groups, int64_t n, int64_t k) {
  (void)total_m; (void)num_groups; (void)n; (void)k;
  return 0;
}

mxfp4_status_t mxfp4_grouped_gemm_nt(const void* a_q, const void* a_s, const void* b_q, const void* b_s,
                                     const int32_t* offsets, int32_t num_groups, int64_t total_m, void* c,
                                     mxfp4_out_t c_type, int64_t n, int64_t k, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  MXFP4_TRY(check_gemm_args(a_q, a_s, b_q, b_s, c, c_type, total_m, n, k));
  if (num_groups < 1 || num_groups > 1024)
    return fail(MXFP4_ERR_INVALID_ARG, "num_groups must be 1..1024 (got %d)", num_groups);
  if (total_m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(offsets, "offsets", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)total_m;
  args.n = (int)n;
  args.k = (int)k;
  args.offsets = offsets;
  args.groups = num_groups;
  const mxfp4::TileKind kind = (total_m / num_groups >= 192) ? mxfp4::kTile256 : mxfp4::kTile128;
  // 256 x 256 tiles go through the persistent loop where it applies: the next
  // tile's first stage loads during a tile's epilogue (about 3 % on a 64-expert
  // MoE layer), with results identical to the one-tile-per-workgroup kernel
  if (kind == mxfp4::kTile256 && mxfp4::gemm_persistent_supported(args))
    return hip_status(mxfp4::launch_grouped_gemm_tile_persistent(args, dev.num_cus, 0, (hipStream_t)stream),
                      "grouped gemm launch");
  return hip_status(mxfp4::launch_grouped_gemm_tile(args, kind, (hipStream_t)stream), "grouped gemm launch");
}

namespace {
// Checks shared by the entry points that take interleaved scales: k % 512 ==
// 0, 16-byte aligned scale arrays, and rows * k/32 < 2^31 for each operand
// (the kernels index a slab of rows with 32-bit byte offsets).
mxfp4_status_t check_interleaved(const void* a_s, const void* b_s, int64_t m, int64_t n, int64_t k) {
  if (k % 512 != 0) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need k %% 512 == 0 (got %lld)", (long long)k);
  if (m * (k / 32) >= ((int64_t)1 << 31) || n * (k / 32) >= ((int64_t)1 << 31))
    return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need rows * k / 32 < 2^31 for each operand");
  if (m > 0) MXFP4_TRY(check_ptr(a_s, "a_s"));
  if (n > 0) MXFP4_TRY(check_ptr(b_s, "b_s"));
  return MXFP4_OK;
}
}  // namespace

mxfp4_status_t mxfp4_scales_interleave(const void* scales, int64_t groups, int64_t rows, int64_t k, void* scales_il,
                                       void* stream) {
  if (groups < 0 || rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  MXFP4_TRY(check_k(k));
  if (k % 512 != 0) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need k %% 512 == 0 (got %lld)", (long long)k);
  if (groups > 0 && rows > ((int64_t)1 << 40) / k / groups) return fail(MXFP4_ERR_INVALID_ARG, "groups * rows * k too large");
  if (groups == 0 || rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(scales, "scales"));
  MXFP4_TRY(check_ptr(scales_il, "scales_il"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_scales_interleave(scales, groups, rows, k, scales_il, (hipStream_t)stream,
                                                    dev.num_cus), "scale interleave launch");
}

mxfp4_status_t mxfp4_quantize_interleaved(const void* x_bf16, int64_t rows, int64_t k, void* q, void* scales_il,
                                          void* stream) {
  if (rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative rows");
  MXFP4_TRY(check_k(k));
  if (k % 512 != 0) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need k %% 512 == 0 (got %lld)", (long long)k);
  if (rows * (k / 32) >= ((int64_t)1 << 31)) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need rows * k / 32 < 2^31");
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(q, "q", 4));
  MXFP4_TRY(check_ptr(scales_il, "scales_il", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_quantize(x_bf16, rows, k, q, scales_il, (hipStream_t)stream, dev.num_cus, true),
                    "interleaved quantize launch");
}

mxfp4_status_t mxfp4_gemm_nt_interleaved(const void* a_q, const void* a_s_il, const void* b_q, const void* b_s_il,
                                         void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream) {
  MXFP4_TRY(check_gemm_args(a_q, a_s_il, b_q, b_s_il, c, c_type, m, n, k));
  MXFP4_TRY(check_interleaved(a_s_il, b_s_il, m, n, k));
  if (m == 0 || n == 0) return MXFP4_OK;
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q;
  args.a_s = (const uint8_t*)a_s_il;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s_il;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  args.scale_il = 1;
  // the tile kernels at every m (the small-M kernels read row-major scales):
  // 256 x 256 tiles once they fill the device, else 128 x 128
  const int64_t tiles256 = ((m + 255) / 256) * ((n + 255) / 256);
  const mxfp4::TileKind kind = tiles256 >= dev.num_cus ? mxfp4::kTile256 : mxfp4::kTile128;
  return hip_status(mxfp4::launch_gemm_tile(args, kind, (hipStream_t)stream), "interleaved gemm launch");
}

mxfp4_status_t mxfp4_grouped_gemm_nt_interleaved(const void* a_q, const void* a_s_il, const void* b_q,
                                                 const void* b_s_il, const int32_t* offsets, int32_t num_groups,
                                                 int64_t total_m, void* c, mxfp4_out_t c_type, int64_t n, int64_t k,
                                                 void* stream) {
  MXFP4_TRY(check_gemm_args(a_q, a_s_il, b_q, b_s_il, c, c_type, total_m, n, k));
  MXFP4_TRY(check_interleaved(a_s_il, b_s_il, total_m, n, k));
  if (num_groups < 1 || num_groups > 1024)
    return fail(MXFP4_ERR_INVALID_ARG, "num_groups must be 1..1024 (got %d)", num_groups);
  if (total_m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(offsets, "offsets", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q;
  args.a_s = (const uint8_t*)a_s_il;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s_il;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)total_m;
  args.n = (int)n;
  args.k = (int)k;
  args.offsets = offsets;
  args.groups = num_groups;
  args.scale_il = 1;
  // the same kernel choice as mxfp4_grouped_gemm_nt
  const mxfp4::TileKind kind = (total_m / num_groups >= 192) ? mxfp4::kTile256 : mxfp4::kTile128;
  if (kind == mxfp4::kTile256 && mxfp4::gemm_persistent_supported(args))
    return hip_status(mxfp4::launch_grouped_gemm_tile_persistent(args, dev.num_cus, 0, (hipStream_t)stream),
                      "interleaved grouped gemm launch");
  return hip_status(mxfp4::launch_grouped_gemm_tile(args, kind, (hipStream_t)stream), "interleaved grouped gemm launch");
}

mxfp4_status_t mxfp8_gemm_w4a8_nt_ex(const void* a_q8, const void* a_s, const void* b_q, const void* b_s, void* c,
                                     mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel,
                                     void* stream) {
  MXFP4_TRY(check_gemm_args(a_q8, a_s, b_q, b_s, c, c_type, m, n, k));
  if (kernel != MXFP4_KERNEL_AUTO && kernel != MXFP4_KERNEL_TILE128 && kernel != MXFP4_KERNEL_STREAM)
    return fail(MXFP4_ERR_INVALID_ARG, "W4A8 kernels: auto, tile128 or stream (got %d)", (int)kernel);
  const bool stream_ok = k % 512 == 0 && ((reinterpret_cast<uintptr_t>(a_s) | reinterpret_cast<uintptr_t>(b_s)) & 15) == 0;
  if (kernel == MXFP4_KERNEL_STREAM && !stream_ok)
    return fail(MXFP4_ERR_INVALID_ARG, "the stream kernel needs k %% 512 == 0 and 16-byte aligned scale arrays");
  if (m == 0 || n == 0) return MXFP4_OK;
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q8;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  const bool use_stream = kernel == MXFP4_KERNEL_STREAM || (kernel == MXFP4_KERNEL_AUTO && m <= 128 && stream_ok);
  if (use_stream) return hip_status(mxfp4::launch_gemm_w4a8_stream(args, (hipStream_t)stream), "w4a8 gemm launch");
  return hip_status(mxfp4::launch_gemm_w4a8_tile(args, (hipStream_t)stream), "w4a8 gemm launch");
}

mxfp4_status_t mxfp8_gemm_w4a8_nt(const void* a_q8, const void* a_s, const void* b_q, const void* b_s, void* c,
                                  mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream) {
  return mxfp8_gemm_w4a8_nt_ex(a_q8, a_s, b_q, b_s, c, c_type, m, n, k, MXFP4_KERNEL_AUTO, stream);
}

mxfp4_status_t mxfp8_gemm_nt_ex(const void* a_q8, const void* a_s, const void* b_q8, const void* b_s, void* c,
                                mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, mxfp4_kernel_t kernel,
                                void* stream) {
  MXFP4_TRY(check_gemm_args(a_q8, a_s, b_q8, b_s, c, c_type, m, n, k));
  // a tile's operand rows span 256 * k bytes of FP8 codes, addressed with 32-bit offsets
  if (k > kMaxK / 2) return fail(MXFP4_ERR_INVALID_ARG, "k too large for MXFP8 operands (%lld > %lld)",
                                 (long long)k, (long long)(kMaxK / 2));
  if (kernel != MXFP4_KERNEL_AUTO && kernel != MXFP4_KERNEL_TILE256 && kernel != MXFP4_KERNEL_TILE128)
    return fail(MXFP4_ERR_INVALID_ARG, "MXFP8 kernels: auto, tile256 or tile128 (got %d)", (int)kernel);
  if (m == 0 || n == 0) return MXFP4_OK;
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q8;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)b_q8;
  args.b_s = (const uint8_t*)b_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  mxfp4::TileKind kind = kernel == MXFP4_KERNEL_TILE128 ? mxfp4::kTile128 : mxfp4::kTile256;
  if (kernel == MXFP4_KERNEL_AUTO && ((m + 255) / 256) * ((n + 255) / 256) < dev.num_cus) kind = mxfp4::kTile128;
  return hip_status(mxfp4::launch_gemm_mxfp8_tile(args, kind, (hipStream_t)stream), "mxfp8 gemm launch");
}

mxfp4_status_t mxfp8_gemm_nt(const void* a_q8, const void* a_s, const void* b_q8, const void* b_s, void* c,
                             mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream) {
  return mxfp8_gemm_nt_ex(a_q8, a_s, b_q8, b_s, c, c_type, m, n, k, MXFP4_KERNEL_AUTO, stream);
}

mxfp4_status_t mxfp8_grouped_gemm_w4a8_nt(const void* a_q8, const void* a_s, const void* b_q, const void* b_s,
                                          const int32_t* offsets, int32_t num_groups, int64_t total_m, void* c,
                                          mxfp4_out_t c_type, int64_t n, int64_t k, void* stream) {
  MXFP4_TRY(check_gemm_args(a_q8, a_s, b_q, b_s, c, c_type, total_m, n, k));
  if (num_groups < 1 || num_groups > 1024)
    return fail(MXFP4_ERR_INVALID_ARG, "num_groups must be 1..1024 (got %d)", num_groups);
  if (total_m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(offsets, "offsets", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q8;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)total_m;
  args.n = (int)n;
  args.k = (int)k;
  args.offsets = offsets;
  args.groups = num_groups;
  // k % 1024 == 0 with 16-byte aligned scale arrays: the persistent tile loop
  // (results identical to the one-tile-per-workgroup kernel)
  if (mxfp4::gemm_persistent_supported(args))
    return hip_status(mxfp4::launch_grouped_gemm_w4a8_tile_persistent(args, dev.num_cus, 0, (hipStream_t)stream),
                      "grouped w4a8 gemm launch");
  return hip_status(mxfp4::launch_grouped_gemm_w4a8_tile(args, (hipStream_t)stream), "grouped w4a8 gemm launch");
}

mxfp4_status_t mxfp8_quantize_interleaved(const void* x_bf16, int64_t rows, int64_t k, void* q8, void* scales_il,
                                          void* stream) {
  if (rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative rows");
  MXFP4_TRY(check_k(k));
  if (k % 512 != 0) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need k %% 512 == 0 (got %lld)", (long long)k);
  if (rows * (k / 32) >= ((int64_t)1 << 31)) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need rows * k / 32 < 2^31");
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(q8, "q8", 8));
  MXFP4_TRY(check_ptr(scales_il, "scales_il", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_quantize_mxfp8(x_bf16, rows, k, q8, scales_il, (hipStream_t)stream, dev.num_cus,
                                                 true), "interleaved mxfp8 quantize launch");
}

namespace {
mxfp4::GemmArgs interleaved_args(const void* a_q, const void* a_s, const void* b_q, const void* b_s, void* c,
                                 mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k) {
  mxfp4::GemmArgs args{};
  args.a_q = (const uint8_t*)a_q;
  args.a_s = (const uint8_t*)a_s;
  args.b_q = (const uint8_t*)b_q;
  args.b_s = (const uint8_t*)b_s;
  args.c = c;
  args.c_f32 = c_type == MXFP4_OUT_F32;
  args.m = (int)m;
  args.n = (int)n;
  args.k = (int)k;
  args.scale_il = 1;
  return args;
}
}  // namespace

mxfp4_status_t mxfp8_gemm_w4a8_nt_interleaved(const void* a_q8, const void* a_s_il, const void* b_q,
                                              const void* b_s_il, void* c, mxfp4_out_t c_type, int64_t m, int64_t n,
                                              int64_t k, void* stream) {
  MXFP4_TRY(check_gemm_args(a_q8, a_s_il, b_q, b_s_il, c, c_type, m, n, k));
  MXFP4_TRY(check_interleaved(a_s_il, b_s_il, m, n, k));
  if (m == 0 || n == 0) return MXFP4_OK;
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  // the 128 x 256 tile kernel at every m (the small-M kernels read row-major scales)
  return hip_status(mxfp4::launch_gemm_w4a8_tile(interleaved_args(a_q8, a_s_il, b_q, b_s_il, c, c_type, m, n, k),
                                                 (hipStream_t)stream), "interleaved w4a8 gemm launch");
}

mxfp4_status_t mxfp8_grouped_gemm_w4a8_nt_interleaved(const void* a_q8, const void* a_s_il, const void* b_q,
                                                      const void* b_s_il, const int32_t* offsets, int32_t num_groups,
                                                      int64_t total_m, void* c, mxfp4_out_t c_type, int64_t n,
                                                      int64_t k, void* stream) {
  MXFP4_TRY(check_gemm_args(a_q8, a_s_il, b_q, b_s_il, c, c_type, total_m, n, k));
  MXFP4_TRY(check_interleaved(a_s_il, b_s_il, total_m, n, k));
  if (num_groups < 1 || num_groups > 1024)
    return fail(MXFP4_ERR_INVALID_ARG, "num_groups must be 1..1024 (got %d)", num_groups);
  if (total_m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(offsets, "offsets", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  mxfp4::GemmArgs args = interleaved_args(a_q8, a_s_il, b_q, b_s_il, c, c_type, total_m, n, k);
  args.offsets = offsets;
  args.groups = num_groups;
  // the same kernel choice as mxfp8_grouped_gemm_w4a8_nt
  if (mxfp4::gemm_persistent_supported(args))
    return hip_status(mxfp4::launch_grouped_gemm_w4a8_tile_persistent(args, dev.num_cus, 0, (hipStream_t)stream),
                      "interleaved grouped w4a8 gemm launch");
  return hip_status(mxfp4::launch_grouped_gemm_w4a8_tile(args, (hipStream_t)stream),
                    "interleaved grouped w4a8 gemm launch");
}

mxfp4_status_t mxfp8_gemm_nt_interleaved(const void* a_q8, const void* a_s_il, const void* b_q8, const void* b_s_il,
                                         void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k, void* stream) {
  MXFP4_TRY(check_gemm_args(a_q8, a_s_il, b_q8, b_s_il, c, c_type, m, n, k));
  if (k > kMaxK / 2) return fail(MXFP4_ERR_INVALID_ARG, "k too large for MXFP8 operands (%lld > %lld)",
                                 (long long)k, (long long)(kMaxK / 2));
  MXFP4_TRY(check_interleaved(a_s_il, b_s_il, m, n, k));
  if (m == 0 || n == 0) return MXFP4_OK;
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  // the same tile choice as mxfp8_gemm_nt
  const mxfp4::TileKind kind = ((m + 255) / 256) * ((n + 255) / 256) < dev.num_cus ? mxfp4::kTile128 : mxfp4::kTile256;
  return hip_status(mxfp4::launch_gemm_mxfp8_tile(interleaved_args(a_q8, a_s_il, b_q8, b_s_il, c, c_type, m, n, k),
                                                  kind, (hipStream_t)stream), "interleaved mxfp8 gemm launch");
}

namespace {
mxfp4_status_t probe_mfma(const void* seed, void* out, int32_t blocks, int32_t iters, bool a_fp8, void* stream) {
  if (blocks < 1 || blocks > 65536) return fail(MXFP4_ERR_INVALID_ARG, "blocks must be 1..65536 (got %d)", blocks);
  if (iters < 1 || iters > (1 << 24)) return fail(MXFP4_ERR_INVALID_ARG, "iters must be 1..2^24 (got %d)", iters);
  MXFP4_TRY(check_ptr(seed, "seed"));
  MXFP4_TRY(check_ptr(out, "out"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_probe_mfma(seed, out, blocks, iters, a_fp8, (hipStream_t)stream),
                    "mfma probe launch");
}
}  // namespace

mxfp4_status_t mxfp4_probe_mfma(const void* seed, void* out, int32_t blocks, int32_t iters, void* stream) {
  return probe_mfma(seed, out, blocks, iters, false, stream);
}

mxfp4_status_t mxfp4_probe_mfma_w4a8(const void* seed, void* out, int32_t blocks, int32_t iters, void* stream) {
  return probe_mfma(seed, out, blocks, iters, true, stream);
}

double mxfp4_probe_mfma_flops(int32_t blocks, int32_t iters) {
  if (blocks < 1 || iters < 1) return 0.0;
  return mxfp4::probe_mfma_flops(blocks, iters);
}

mxfp4_status_t mxfp4_probe_read(const void* src, int64_t bytes, void* out, int32_t blocks, void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40))
    return fail(MXFP4_ERR_INVALID_ARG, "bytes must be a positive multiple of 16, at most 2^40 (got %lld)",
                (long long)bytes);
  if (blocks < 1 || blocks > 65536) return fail(MXFP4_ERR_INVALID_ARG, "blocks must be 1..65536 (got %d)", blocks);
  MXFP4_TRY(check_ptr(src, "src"));
  MXFP4_TRY(check_ptr(out, "out", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_probe_read(src, bytes, out, blocks, (hipStream_t)stream), "read probe launch");
}

// ---------------------------------------------------------------------------
// MoE steps (include/mxfp4_moe.h)
// ---------------------------------------------------------------------------

mxfp4_status_t mxfp4_moe_route(const float* logits, int64_t tokens, int32_t experts, int32_t top_k,
                               int32_t* topk_ids, float* topk_weights, void* stream) {
  if (tokens < 0 || tokens > ((int64_t)1 << 28)) return fail(MXFP4_ERR_INVALID_ARG, "tokens must be 0..2^28 (got %lld)", (long long)tokens);
  if (experts < 1 || experts > mxfp4::kMoeMaxRouteExperts)
    return fail(MXFP4_ERR_INVALID_ARG, "experts must be 1..%d (got %d)", mxfp4::kMoeMaxRouteExperts, experts);
  if (top_k < 1 || top_k > mxfp4::kMoeMaxTopK || top_k > experts)
    return fail(MXFP4_ERR_INVALID_ARG, "top_k must be 1..min(%d, experts) (got %d)", mxfp4::kMoeMaxTopK, top_k);
  if (tokens == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(logits, "logits", 4));
  MXFP4_TRY(check_ptr(topk_ids, "topk_ids", 4));
  MXFP4_TRY(check_ptr(topk_weights, "topk_weights", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_moe_route(logits, (int)tokens, experts, top_k, topk_ids, topk_weights,
                                            (hipStream_t)stream), "moe route launch");
}

mxfp4_status_t mxfp4_moe_permute(const int32_t* topk_ids, int64_t tokens, int32_t experts, int32_t top_k,
                                 int32_t* offsets, int32_t* row_token, int32_t* token_rows, void* stream) {
  if (tokens < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative tokens");
  if (experts < 1 || experts > 1024) return fail(MXFP4_ERR_INVALID_ARG, "experts must be 1..1024 (got %d)", experts);
  if (top_k < 1 || top_k > 256) return fail(MXFP4_ERR_INVALID_ARG, "top_k must be 1..256 (got %d)", top_k);
  if (tokens > ((int64_t)1 << 30) / top_k) return fail(MXFP4_ERR_INVALID_ARG, "tokens * top_k too large");
  MXFP4_TRY(check_ptr(offsets, "offsets", 4));
  if (tokens > 0) {
    MXFP4_TRY(check_ptr(topk_ids, "topk_ids", 4));
    MXFP4_TRY(check_ptr(row_token, "row_token", 4));
    MXFP4_TRY(check_ptr(token_rows, "token_rows", 4));
  }
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_moe_permute(topk_ids, (int)(tokens * top_k), top_k, experts, offsets, row_token,
                                              token_rows, (hipStream_t)stream), "moe permute launch");
}

namespace {
mxfp4_status_t moe_quantize_scatter(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                    const int32_t* token_rows, int64_t total_rows, void* q, void* scales,
                                    bool fp8, void* stream, bool interleaved = false) {
  if (tokens < 0 || total_rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  MXFP4_TRY(check_k(k));
  if (top_k < 1 || top_k > 256) return fail(MXFP4_ERR_INVALID_ARG, "top_k must be 1..256 (got %d)", top_k);
  if (tokens > ((int64_t)1 << 30) / (k / 32)) return fail(MXFP4_ERR_INVALID_ARG, "tokens * k / 32 too large");
  if (total_rows >= ((int64_t)1 << 31)) return fail(MXFP4_ERR_INVALID_ARG, "total_rows too large");
  if (interleaved) {
    if (k % 512 != 0) return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need k %% 512 == 0 (got %lld)", (long long)k);
    if (total_rows * (k / 32) >= ((int64_t)1 << 31))
      return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need total_rows * k / 32 < 2^31");
  }
  if (tokens == 0 || total_rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(token_rows, "token_rows", 4));
  MXFP4_TRY(check_ptr(q, fp8 ? "q8" : "q", fp8 ? 8 : 4));
  MXFP4_TRY(check_ptr(scales, "scales", 1));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_moe_quantize_scatter(x_bf16, (int)tokens, (int)k, top_k, token_rows,
                                                       (int)total_rows, q, scales, fp8, (hipStream_t)stream,
                                                       dev.num_cus, interleaved), "moe quantize-scatter launch");
}
}  // namespace

mxfp4_status_t mxfp4_moe_quantize_scatter(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                          const int32_t* token_rows, int64_t total_rows, void* q, void* scales,
                                          void* stream) {
  return moe_quantize_scatter(x_bf16, tokens, k, top_k, token_rows, total_rows, q, scales, false, stream);
}

mxfp4_status_t mxfp4_moe_quantize_scatter_interleaved(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                                      const int32_t* token_rows, int64_t total_rows, void* q,
                                                      void* scales_il, void* stream) {
  return moe_quantize_scatter(x_bf16, tokens, k, top_k, token_rows, total_rows, q, scales_il, false, stream, true);
}

mxfp4_status_t mxfp8_moe_quantize_scatter_interleaved(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                                      const int32_t* token_rows, int64_t total_rows, void* q8,
                                                      void* scales_il, void* stream) {
  return moe_quantize_scatter(x_bf16, tokens, k, top_k, token_rows, total_rows, q8, scales_il, true, stream, true);
}

mxfp4_status_t mxfp8_moe_quantize_scatter(const void* x_bf16, int64_t tokens, int64_t k, int32_t top_k,
                                          const int32_t* token_rows, int64_t total_rows, void* q8, void* scales,
                                          void* stream) {
  return moe_quantize_scatter(x_bf16, tokens, k, top_k, token_rows, total_rows, q8, scales, true, stream);
}

mxfp4_status_t mxfp4_moe_combine(const void* y_bf16, int64_t total_rows, int64_t n, const int32_t* token_rows,
                                 const float* topk_weights, int64_t tokens, int32_t top_k, void* out,
                                 mxfp4_out_t out_type, void* stream) {
  if (tokens < 0 || total_rows < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "n too large");
  if (total_rows >= ((int64_t)1 << 31)) return fail(MXFP4_ERR_INVALID_ARG, "total_rows too large");
  if (top_k < 1 || top_k > 256) return fail(MXFP4_ERR_INVALID_ARG, "top_k must be 1..256 (got %d)", top_k);
  if (out_type != MXFP4_OUT_BF16 && out_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)out_type);
  if (n > 0 && tokens >= ((int64_t)1 << 31) / ((n + 7) / 8)) return fail(MXFP4_ERR_INVALID_ARG, "tokens * ceil(n / 8) too large");
  if (tokens == 0 || n == 0) return MXFP4_OK;
  const bool f32 = out_type == MXFP4_OUT_F32;
  MXFP4_TRY(check_ptr(y_bf16, "y_bf16", 2));
  MXFP4_TRY(check_ptr(token_rows, "token_rows", 4));
  MXFP4_TRY(check_ptr(topk_weights, "topk_weights", 4));
  MXFP4_TRY(check_ptr(out, "out", f32 ? 4 : 2));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  const bool vec = n % 8 == 0 && aligned16(y_bf16) && aligned16(out);
  return hip_status(mxfp4::launch_moe_combine(y_bf16, (int)total_rows, (int)n, token_rows, topk_weights, (int)tokens,
                                              top_k, out, f32, vec, (hipStream_t)stream), "moe combine launch");
}

// ---------------------------------------------------------------------------
// Fused producers (include/mxfp4_producers.h)
// ---------------------------------------------------------------------------

namespace {
mxfp4_status_t rmsnorm_quantize(const void* x_bf16, const void* residual_bf16, const void* gamma_bf16, float eps,
                                int64_t rows, int64_t k, void* residual_out_bf16, void* y_bf16, void* q, void* scales,
                                int layout, void* stream) {
  const bool prepacked = layout == mxfp4::kLayoutPrepacked;
  // one 256-thread workgroup per row (prepacked: per row of whole 64-row panels)
  if (rows < 0 || rows > ((int64_t)1 << 24)) return fail(MXFP4_ERR_INVALID_ARG, "rows must be 0..2^24 (got %lld)", (long long)rows);
  MXFP4_TRY(check_k(k));
  if (k > 256 * 8 * mxfp4::kNormMaxSlots)
    return fail(MXFP4_ERR_INVALID_ARG, "k must be at most %d for the RMSNorm producer (got %lld)",
                256 * 8 * mxfp4::kNormMaxSlots, (long long)k);
  if (layout != mxfp4::kLayoutRowMajor && k % 512)
    return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (layout == mxfp4::kLayoutInterleaved && rows * (k / 32) >= ((int64_t)1 << 31))
    return fail(MXFP4_ERR_INVALID_ARG, "interleaved scales need rows * k / 32 < 2^31");
  if (!(eps >= 0.0f) || eps == __builtin_huge_valf()) return fail(MXFP4_ERR_INVALID_ARG, "eps must be finite and non-negative");
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(gamma_bf16, "gamma_bf16"));
  MXFP4_TRY(check_ptr(q, prepacked ? "ap_q" : "q", prepacked ? 16 : 4));
  MXFP4_TRY(check_ptr(scales, prepacked ? "ap_s" : "scales", 1));
  if (residual_bf16) MXFP4_TRY(check_ptr(residual_bf16, "residual_bf16"));
  if (residual_out_bf16) {
    if (!residual_bf16) return fail(MXFP4_ERR_INVALID_ARG, "residual_out_bf16 needs residual_bf16");
    MXFP4_TRY(check_ptr(residual_out_bf16, "residual_out_bf16"));
  }
  if (y_bf16) MXFP4_TRY(check_ptr(y_bf16, "y_bf16"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_rmsnorm_quantize(x_bf16, residual_bf16, gamma_bf16, eps, (int)rows, (int)k,
                                                   residual_out_bf16, y_bf16, q, scales, layout,
                                                   (hipStream_t)stream),
                    "rmsnorm quantize launch");
}

mxfp4_status_t swiglu_quantize(const void* gate_bf16, const void* up_bf16, int64_t ld, int64_t rows, int64_t k,
                               void* y_bf16, void* q, void* scales, int layout, void* stream) {
  const bool prepacked = layout == mxfp4::kLayoutPrepacked;
  if (rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative rows");
  MXFP4_TRY(check_k(k));
  if (layout != mxfp4::kLayoutRowMajor && k % 512)
    return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (ld < k || ld % 8 != 0) return fail(MXFP4_ERR_INVALID_ARG, "ld must be a multiple of 8 and at least k (got %lld)", (long long)ld);
  if ((rows + 63) / 64 * 64 > ((int64_t)1 << 30) / (k / 32)) return fail(MXFP4_ERR_INVALID_ARG, "rows * k / 32 too large");
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(gate_bf16, "gate_bf16"));
  MXFP4_TRY(check_ptr(up_bf16, "up_bf16"));
  MXFP4_TRY(check_ptr(q, prepacked ? "ap_q" : "q", prepacked ? 16 : 4));
  MXFP4_TRY(check_ptr(scales, prepacked ? "ap_s" : "scales", 1));
  if (y_bf16) MXFP4_TRY(check_ptr(y_bf16, "y_bf16"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_swiglu_quantize(gate_bf16, up_bf16, ld, (int)rows, (int)k, y_bf16, q, scales,
                                                  layout, (hipStream_t)stream, dev.num_cus),
                    "swiglu quantize launch");
}
}  // namespace

mxfp4_status_t mxfp4_rmsnorm_quantize(const void* x_bf16, const void* residual_bf16, const void* gamma_bf16,
                                      float eps, int64_t rows, int64_t k, void* residual_out_bf16, void* y_bf16,
                                      void* q, void* scales, void* stream) {
  return rmsnorm_quantize(x_bf16, residual_bf16, gamma_bf16, eps, rows, k, residual_out_bf16, y_bf16, q, scales,
                          mxfp4::kLayoutRowMajor, stream);
}

mxfp4_status_t mxfp4_rmsnorm_quantize_interleaved(const void* x_bf16, const void* residual_bf16,
                                                  const void* gamma_bf16, float eps, int64_t rows, int64_t k,
                                                  void* residual_out_bf16, void* y_bf16, void* q, void* scales_il,
                                                  void* stream) {
  return rmsnorm_quantize(x_bf16, residual_bf16, gamma_bf16, eps, rows, k, residual_out_bf16, y_bf16, q, scales_il,
                          mxfp4::kLayoutInterleaved, stream);
}

mxfp4_status_t mxfp4_rmsnorm_quantize_prepacked(const void* x_bf16, const void* residual_bf16,
                                                const void* gamma_bf16, float eps, int64_t rows, int64_t k,
                                                void* residual_out_bf16, void* y_bf16, void* ap_q, void* ap_s,
                                                void* stream) {
  return rmsnorm_quantize(x_bf16, residual_bf16, gamma_bf16, eps, rows, k, residual_out_bf16, y_bf16, ap_q, ap_s,
                          mxfp4::kLayoutPrepacked, stream);
}

mxfp4_status_t mxfp4_swiglu_quantize(const void* gate_bf16, const void* up_bf16, int64_t ld, int64_t rows,
                                     int64_t k, void* y_bf16, void* q, void* scales, void* stream) {
  return swiglu_quantize(gate_bf16, up_bf16, ld, rows, k, y_bf16, q, scales, mxfp4::kLayoutRowMajor, stream);
}

mxfp4_status_t mxfp4_swiglu_quantize_interleaved(const void* gate_bf16, const void* up_bf16, int64_t ld,
                                                 int64_t rows, int64_t k, void* y_bf16, void* q, void* scales_il,
                                                 void* stream) {
  return swiglu_quantize(gate_bf16, up_bf16, ld, rows, k, y_bf16, q, scales_il, mxfp4::kLayoutInterleaved, stream);
}

mxfp4_status_t mxfp4_swiglu_quantize_prepacked(const void* gate_bf16, const void* up_bf16, int64_t ld, int64_t rows,
                                               int64_t k, void* y_bf16, void* ap_q, void* ap_s, void* stream) {
  return swiglu_quantize(gate_bf16, up_bf16, ld, rows, k, y_bf16, ap_q, ap_s, mxfp4::kLayoutPrepacked, stream);
}

// ---------------------------------------------------------------------------
// NVFP4 (include/nvfp4.h)
// ---------------------------------------------------------------------------

mxfp4_status_t nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t k, void* q, void* scales,
                              float* global_scales, void* stream) {
  // one 256-thread workgroup per row: a launch holds fewer than 2^32 threads
  if (rows < 0 || rows > ((int64_t)1 << 24)) return fail(MXFP4_ERR_INVALID_ARG, "rows must be 0..2^24 (got %lld)", (long long)rows);
  MXFP4_TRY(check_k(k));
  if (k > 256 * 8 * mxfp4::kNormMaxSlots)
    return fail(MXFP4_ERR_INVALID_ARG, "k must be at most %d for the NVFP4 quantizer (got %lld)",
                256 * 8 * mxfp4::kNormMaxSlots, (long long)k);
  if (rows == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(x_bf16, "x_bf16"));
  MXFP4_TRY(check_ptr(q, "q", 4));
  MXFP4_TRY(check_ptr(scales, "scales", 1));
  MXFP4_TRY(check_ptr(global_scales, "global_scales", 4));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_nvfp4_quantize(x_bf16, (int)rows, (int)k, q, scales, global_scales,
                                                 (hipStream_t)stream), "nvfp4 quantize launch");
}

mxfp4_status_t nvfp4_gemm_nt(const void* a_q, const void* a_s, const float* a_gs, const void* b_q, const void* b_s,
                             const float* b_gs, void* c, mxfp4_out_t c_type, int64_t m, int64_t n, int64_t k,
                             void* stream) {
  if (m < 0 || n < 0) return fail(MXFP4_ERR_INVALID_ARG, "negative size");
  if (m > kMaxDim || n > kMaxDim) return fail(MXFP4_ERR_INVALID_ARG, "m or n too large");
  MXFP4_TRY(check_k(k));
  if (k % 64 != 0) return fail(MXFP4_ERR_INVALID_ARG, "k must be a multiple of 64 for the NVFP4 GEMM (got %lld)", (long long)k);
  if (c_type != MXFP4_OUT_BF16 && c_type != MXFP4_OUT_F32)
    return fail(MXFP4_ERR_INVALID_ARG, "unknown output type %d", (int)c_type);
  if (m == 0 || n == 0) return MXFP4_OK;
  MXFP4_TRY(check_ptr(a_q, "a_q"));
  MXFP4_TRY(check_ptr(a_s, "a_s", 4));
  MXFP4_TRY(check_ptr(a_gs, "a_gs", 4));
  MXFP4_TRY(check_ptr(b_q, "b_q"));
  MXFP4_TRY(check_ptr(b_s, "b_s", 4));
  MXFP4_TRY(check_ptr(b_gs, "b_gs", 4));
  MXFP4_TRY(check_ptr(c, "c"));
  DeviceInfo dev;
  MXFP4_TRY(current_device(dev));
  return hip_status(mxfp4::launch_nvfp4_gemm(a_q, a_s, a_gs, b_q, b_s, b_gs, c, c_type == MXFP4_OUT_F32, (int)m,
                                             (int)n, (int)k, (hipStream_t)stream), "nvfp4 gemm launch");
}

}  // extern "C"
