// Host-side launch functions of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

struct GemmArgs {
  const uint8_t* a_q;      // [m, k/2]
  const uint8_t* a_s;      // [m, k/32], or interleaved [k/512, m, 16]
  const uint8_t* b_q;      // [n, k/2] (grouped: [groups, n, k/2])
  const uint8_t* b_s;      // [n, k/32] (grouped: [groups, n, k/32]), or interleaved [(groups,) k/512, n, 16]
  void* c;                 // [m, n]
  int c_f32;               // 0: bf16 output, 1: fp32 output
  int m, n, k;             // grouped: m = total_m
  const int32_t* offsets;  // grouped only: device [groups + 1]
  int groups;              // grouped only
  int scale_il;            // 1: both scale arrays interleaved (tile kernels' copy path only)
};

// One HIP launch holds at most 2^32 - 1 threads.  Grid sizes are computed in
// 64 bits and checked with this before every launch, so a problem too large
// for one launch is refused (hipErrorInvalidConfiguration) instead of running
// a truncated grid.
inline bool grid_fits(int64_t blocks, int threads) {
  return blocks >= 1 && blocks * threads <= (int64_t)0xFFFFFFFF;
}

// Tile kernels (TILE256: 256x256 output tiles, TILE128: 128x128 output tiles).
enum TileKind { kTile256 = 0, kTile128 = 1 };

// interleaved: scale bytes in the tile GEMMs' interleaved layout [k/512, rows, 16]
// (k % 512 == 0, rows * k/32 < 2^31; hipErrorInvalidValue otherwise).
hipError_t launch_quantize(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                           hipStream_t stream, int num_cus, bool interleaved = false);
// Scale bytes [groups, rows, k/32] rearranged into [groups, k/512, rows, 16].
hipError_t launch_scales_interleave(const void* scales, int64_t groups, int64_t rows, int64_t k, void* out,
                                    hipStream_t stream, int num_cus);
// The same codes and scale bytes stored in the prepacked GEMM operand layout
// (k % 512 == 0; rows up to the next multiple of 64 written as zero blocks).
hipError_t launch_quantize_prepacked(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                                     hipStream_t stream, int num_cus);
hipError_t launch_quantize_mxfp8(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                                 hipStream_t stream, int num_cus, bool interleaved = false);
// MXFP8 codes and scales stored in the FP8 prepacked operand layout (k % 512 == 0;
// rows up to the next multiple of 64 written as zero blocks).
hipError_t launch_quantize_mxfp8_prepacked(const void* x, int64_t rows, int64_t k, void* q, void* scales,
                                           hipStream_t stream, int num_cus);

hipError_t launch_gemm_tile(const GemmArgs& args, TileKind kind, hipStream_t stream);

hipError_t launch_grouped_gemm_tile(const GemmArgs& args, TileKind kind, hipStream_t stream);

// Persistent 256x256 tile kernels: at most one workgroup per compute unit
// (capped by max_wgs when > 0), each looping over its tiles and copying the
// next tile's first stage during the current tile's last stages and epilogue.
// Need k % 1024 == 0 and 16-byte aligned scale arrays (gemm_persistent_supported).
bool gemm_persistent_supported(const GemmArgs& args);
hipError_t launch_gemm_tile_persistent(const GemmArgs& args, int num_cus, int max_wgs, hipStream_t stream);
hipError_t launch_grouped_gemm_tile_persistent(const GemmArgs& args, int num_cus, int max_wgs, hipStream_t stream);

// W4A8 tile kernels: A in MXFP8 (a_q is [m, k] E4M3 codes), B in MXFP4;
// 128 x 256 output tiles.
hipError_t launch_gemm_w4a8_tile(const GemmArgs& args, hipStream_t stream);
hipError_t launch_grouped_gemm_w4a8_tile(const GemmArgs& args, hipStream_t stream);
// The grouped W4A8 GEMM through the persistent tile loop (128 x 256 tiles;
// needs what gemm_persistent_supported checks).
hipError_t launch_grouped_gemm_w4a8_tile_persistent(const GemmArgs& args, int num_cus, int max_wgs,
                                                    hipStream_t stream);

// MXFP8 x MXFP8 tile kernels (a_q and b_q are [rows, k] E4M3 codes): 256 x 256
// or 128 x 128 output tiles over 128-K stages; a tile's operand rows span at
// most 256 * k bytes, so k <= 2^23.
hipError_t launch_gemm_mxfp8_tile(const GemmArgs& args, TileKind kind, hipStream_t stream);

// Bandwidth path for m <= 128: 64- or 32-column tiles, K split over the 4 waves
// of a workgroup and, when splits > 1, over `splits` workgroups per tile with
// fp32 partials and per-tile arrival counters in `workspace`.
size_t splitk_workspace_bytes(int m, int n, int k, int splits);
int splitk_max_tiles();   // largest ceil(n / 64) that splits > 1 supports
int splitk_auto_splits(int m, int n, int k, int num_cus);
hipError_t launch_gemm_splitk(const GemmArgs& args, int splits, void* workspace,
                              hipStream_t stream, int num_cus);
// Zeroes the per-tile arrival counters at the start of a split-K workspace
// (every launch with splits > 1 leaves them at zero again).
hipError_t launch_splitk_clear_counters(void* workspace, hipStream_t stream);

// Small-M weight-streaming kernel: 64-column tiles over the whole K with the
// 4 waves of a workgroup splitting each 256-K stage by k-step; needs
// k % 512 == 0 and 16-byte aligned scale arrays (hipErrorInvalidValue otherwise).
bool stream_supported(const GemmArgs& args);
hipError_t launch_gemm_stream(const GemmArgs& args, hipStream_t stream);
// The same with A in MXFP8 (W4A8); M tiles of 32 or 64 rows.
hipError_t launch_gemm_w4a8_stream(const GemmArgs& args, hipStream_t stream);

// The same on a prepacked weight (include/mxfp4.h, mxfp4_prepack_weight): B is
// loaded straight into registers; A as in launch_gemm_stream.
void prepacked_sizes(int64_t n, int64_t k, int64_t* code_bytes, int64_t* scale_bytes);
hipError_t launch_prepack_weight(const uint8_t* b_q, const uint8_t* b_s, int n, int k, uint8_t* bp_q, uint8_t* bp_s,
                                 hipStream_t stream);
hipError_t launch_gemm_stream_prepacked(const GemmArgs& args, hipStream_t stream);
// W4A8 on a prepacked weight: A in MXFP8 (a_q [m, k] E4M3 codes) through the
// LDS ring, B prepacked into registers; k % 512 == 0, 16-byte aligned scales.
hipError_t launch_gemm_w4a8_stream_prepacked(const GemmArgs& args, hipStream_t stream);
// Both operands prepacked (a_q / a_s and b_q / b_s in the prepacked layout):
// no LDS in the main loop.  splits > 1: each output tile's K is cut into that
// many ranges (fewer when K has fewer 512-K pairs) reduced through
// `workspace` (pp_workspace_bytes; zero-filled before first use, left
// zero-filled); hipErrorInvalidValue when the shape has more output tiles
// than the workspace's counter region holds.
hipError_t launch_gemm_both_prepacked(const GemmArgs& args, int splits, void* workspace, hipStream_t stream);
// W4A8 on both operands prepacked: A in the FP8 prepacked layout, B in the MXFP4
// prepacked layout (k % 512 == 0; bit-identical to launch_gemm_w4a8_stream_prepacked).
hipError_t launch_gemm_w4a8_both_prepacked(const GemmArgs& args, hipStream_t stream);
// The K ranges a request for `splits` gives: ranges of ceil(pairs / splits)
// 512-K pairs, rounded up to a multiple of 4 above 4 (at most `splits`, none
// empty).
int pp_effective_splits(int k, int splits);
// The automatic choice: enough ranges to give most compute units a workgroup.
int pp_auto_splits(int m, int n, int k, int num_cus);
// Workspace bytes for `splits` (0 when the effective count is 1 or the shape
// has too many output tiles for split-K).
size_t pp_workspace_bytes(int m, int n, int k, int splits);

// MoE steps around the grouped GEMM (include/mxfp4_moe.h).
constexpr int kMoeMaxTopK = 8;          // routing: experts per token
constexpr int kMoeMaxRouteExperts = 256;  // routing: four logits per lane of a wave
hipError_t launch_moe_route(const float* logits, int tokens, int experts, int top_k, int32_t* ids, float* weights,
                            hipStream_t stream);
hipError_t launch_moe_permute(const int32_t* ids, int n, int top_k, int experts, int32_t* offsets,
                              int32_t* row_token, int32_t* token_rows, hipStream_t stream);
// interleaved: the scale bytes in the interleaved layout [k/512, total_rows, 16]
// (k % 512 == 0, total_rows * k/32 < 2^31).
hipError_t launch_moe_quantize_scatter(const void* x, int tokens, int k, int top_k, const int32_t* token_rows,
                                       int total_rows, void* q, void* scales, bool fp8, hipStream_t stream,
                                       int num_cus, bool interleaved = false);
hipError_t launch_moe_combine(const void* y, int total_rows, int n, const int32_t* token_rows, const float* weights,
                              int tokens, int top_k, void* out, bool f32_out, bool vec, hipStream_t stream);

// Fused producers emitting MXFP4 activations (include/mxfp4_producers.h).
constexpr int kNormMaxSlots = 16;   // RMSNorm rows: k <= 256 threads * 8 elements * 16 = 32768
// Where a producer writes its MXFP4 bytes: row-major codes and scales; codes and
// scales in the prepacked operand layout; or row-major codes with interleaved
// scales [k/512, rows, 16] (the last two need k % 512 == 0, interleaved also
// rows * k/32 < 2^31).
enum ProducerLayout { kLayoutRowMajor = 0, kLayoutPrepacked = 1, kLayoutInterleaved = 2 };
hipError_t launch_rmsnorm_quantize(const void* x, const void* residual, const void* gamma, float eps, int rows, int k,
                                   void* h_out, void* y_out, void* q, void* scales, int layout,
                                   hipStream_t stream);
hipError_t launch_swiglu_quantize(const void* gate, const void* up, int64_t ld, int rows, int k, void* y_out, void* q,
                                  void* scales, int layout, hipStream_t stream, int num_cus);

// NVFP4 (include/nvfp4.h): quantization (k <= 32768, one workgroup per row) and
// the dequantizing NT GEMM on the BF16 MFMA (k % 64 == 0).
hipError_t launch_nvfp4_quantize(const void* x, int rows, int k, void* q, void* scales, float* gs,
                                 hipStream_t stream);
hipError_t launch_nvfp4_gemm(const void* a_q, const void* a_s, const float* a_gs, const void* b_q, const void* b_s,
                             const float* b_gs, void* c, bool c_f32, int m, int n, int k, hipStream_t stream);

// Measurement probes (include/mxfp4_probe.h).
double probe_mfma_flops(int blocks, int iters);
hipError_t launch_probe_mfma(const void* seed, void* out, int blocks, int iters, bool a_fp8, hipStream_t stream);
hipError_t launch_probe_read(const void* src, int64_t bytes, void* out, int blocks, hipStream_t stream);

}  // namespace mxfp4
