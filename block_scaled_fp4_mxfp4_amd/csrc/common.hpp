// Device-side helpers shared by the gfx950 kernels of the MXFP4 library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

#define MXFP4_LDS __attribute__((address_space(3)))

// Element formats of the scaled f8f6f4 MFMA: 0 selects FP8 E4M3 for an
// operand, 4 selects FP4 E2M1.
constexpr int kMfmaFmtFp8 = 0;
constexpr int kMfmaFmtFp4 = 4;

// s_waitcnt immediate on gfx9: wait until at most `n` vector-memory operations
// are outstanding; the export and LDS/scalar counters are left unconstrained.
__device__ __forceinline__ constexpr int waitcnt_vm_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}
#define MXFP4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(::mxfp4::waitcnt_vm_imm(n))
// wait for every outstanding LDS/scalar-memory operation
#define MXFP4_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8))

// fp32 -> bf16 with round-to-nearest-even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Direct global -> LDS copies (gfx950): lane i's bytes land at lds_base + i * size,
// lds_base must be wave-uniform.
__device__ __forceinline__ void g2lds_16(const void* gptr, MXFP4_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}
__device__ __forceinline__ void g2lds_4(const void* gptr, MXFP4_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 4, 0, 0);
}

// Raw buffer resource over `bytes` bytes from `base` (gfx9 descriptor word 3:
// 32-bit data format, no swizzle, no stride).  Loads at offsets past `bytes`
// return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes at voffset + soffset in the
// buffer land at lds_base + 16 * i.  The buffer base and soffset stay in scalar
// registers, so each copy needs one 32-bit vector register and no address
// arithmetic.  lds_base must be wave-uniform.
__device__ __forceinline__ void buf2lds_16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset,
                                           MXFP4_LDS void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voffset, soffset, 0, 0);
}

// One 32x32x64 block-scaled FP4 MFMA step: D += (A scaled) x (B scaled)^T.
// Lane l supplies row (l % 32), K-block (l / 32): 16 bytes of codes and the
// E8M0 byte selected by OPSEL out of its 32-bit scale register.
template <int OPSEL>
__device__ __forceinline__ v16f mfma32_fp4(v4i a, v4i b, v16f acc, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  v8i b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc, kMfmaFmtFp4, kMfmaFmtFp4,
                                                         OPSEL, sa, OPSEL, sb);
}

// The same step with the second operand in FP8 E4M3: lane l supplies 32
// codes of row (l % 32), K [16h, 16h + 16) in its first four registers and
// [32 + 16h, 48 + 16h) in the last four (h = l / 32); its scale byte still
// covers K-block h.  With an FP8 operand the MFMA runs at the FP8 rate.
template <int OPSEL>
__device__ __forceinline__ v16f mfma32_fp4_fp8(v4i a, v8i b, v16f acc, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, acc, kMfmaFmtFp4, kMfmaFmtFp8,
                                                         OPSEL, sa, OPSEL, sb);
}

// The same step with both operands in FP8 E4M3 (32 codes per lane in the
// interleaved order above), at the FP8 rate.
template <int OPSEL>
__device__ __forceinline__ v16f mfma32_fp8(v8i a, v8i b, v16f acc, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, kMfmaFmtFp8, kMfmaFmtFp8, OPSEL, sa, OPSEL, sb);
}

// The prepacked operand layout (include/mxfp4.h, mxfp4_prepacked_weight_size):
// for 32-element block kb of row r of an operand with `pairs` 512-K pairs per
// row, the index of its first 4-byte code word (its four words are
// consecutive) and of its scale byte.
__device__ __forceinline__ void prepacked_index(int64_t r, int kb, int pairs, int64_t& word, int64_t& sbyte) {
  const int64_t panel = r / 64;
  const int rr = (int)(r - panel * 64);
  const int j = rr >> 5, t = kb >> 4, s = (kb >> 3) & 1, w = (kb >> 1) & 3;
  const int l = (rr & 31) + 32 * (kb & 1);
  const int64_t blk = panel * pairs + t;
  word = (blk * 16384 + w * 4096 + (2 * s + j) * 1024 + l * 16) / 4;
  sbyte = blk * 1024 + w * 256 + l * 4 + 2 * s + j;
}

// Tile index -> (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs of MI355X, each XCD with a private L2.  When the tile count is a
// multiple of 8, consecutive logical tiles are placed on one XCD; logical tiles
// then walk `group_m` tile rows before moving one tile column, so an XCD's
// tiles share a few A and B panels in its L2.
// Logical tile t -> (tile_m, tile_n): logical tiles walk `group_m` tile rows
// before moving one tile column.
__device__ __forceinline__ void tile_order(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int gsize = min(tiles_m - first_m, group_m);
  const int r = t - g * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int t = bid;
  if ((total & 7) == 0) {
    const int per_xcd = total >> 3;
    t = (bid & 7) * per_xcd + (bid >> 3);
  }
  tile_order(t, tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace mxfp4
