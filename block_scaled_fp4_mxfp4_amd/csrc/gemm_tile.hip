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
//    by op_sel).  The block scale is applied inside the MFMA: no dequantized
//    operand ever exists; packed bytes go HBM -> LDS -> VGPR unchanged.
//  * The MFMA's first operand is fed from B and its second from A, so the
//    result lands transposed: lane l holds output row (l % 32) and four runs of
//    four consecutive output columns.
//  * A stage covers 256 K elements = 128 code bytes per row, so each
//    buffer_load_dwordx4 ... lds (64 lanes x 16 bytes, straight into LDS)
//    moves 8 whole 128-byte rows; 64-byte row pieces measured about half the
//    per-CU copy rate.  Two code stages are in flight (2 x 64 KiB for 256x256).
//    The copies go through buffer resources over the tile's operand rows: the
//    base and the stage offset live in scalar registers and each copy needs
//    one 32-bit vector register, which keeps the 8-wave main loop free of
//    spills (64-bit global addresses measured 3-5 % slower and spilled once the
//    loop was specialized below).
//  * Scale bytes travel separately: one 16-byte piece per row covers two
//    stages (512 K), so the scale copy costs an eighth of the code copy's
//    requests instead of one 4-byte request per row per stage.  Two scale
//    groups are in flight.
//  * LDS rows are 128 bytes = eight 16-byte chunks; logical chunk c of row r
//    sits at chunk c ^ ((r >> 1) & 7), which makes the ds_read_b128 of 32
//    consecutive rows at one chunk conflict-free (measured on the device).
//  * Pipeline: iteration kt computes stage kt in four 64-deep k-steps,
//    reading the next k-step's fragments while the current MFMAs run.  Before
//    the last k-step every wave waits for its copies of stage kt+1 and passes
//    one barrier; then the buffer of stage kt is free, the copies of stage
//    kt+2 go into it, and stage kt+1's first fragments are read while the last
//    MFMAs of stage kt run.
//  * Waves form a 2 x WGN grid over the tile, each owning a (BM/2) x (BN/WGN)
//    sub-tile of 32x32 MFMA blocks.  256x256 tiles use 8 waves (2 per SIMD,
//    128x64 each, 256 registers per wave): with one wave per SIMD every stall
//    of its in-order instruction stream (a fragment wait, a copy or read
//    stuck at issue, a barrier) idled that SIMD's matrix unit, and counters
//    showed waves waiting on instruction issue about half of the time; a
//    second wave fills those gaps.  Wave w runs on SIMD w % 4 and the two
//    waves of a SIMD sit in different wave rows.
//  * Row blocks past the tile's last stored row (an expert's last rows, a
//    ragged M) are skipped: each wave runs a main loop specialized for its
//    number of 32-row MFMA blocks that hold stored rows.
//  * Copies of the next stage are issued spread over the MFMAs of the last
//    k-step rather than in one burst.
//  * Workgroup -> tile mapping is XCD-aware (see tile_coords in common.hpp);
//    the grouped kernel splits its real tiles evenly over the XCDs.
//
// W4A8 (MXFP8 activations x MXFP4 weights, "fp4_quantization" page: the
// block-scaled matmul also takes MXFP8 operands; quantize_dynamic_scaled_fp4fp8
// produces them): the same kernel with A in FP8 E4M3, one code byte per
// element, on the same MFMA with A's format set to FP8.
//  * Lane l then supplies 32 bytes of A for row l % 32: with h = l / 32, K
//    [16h, 16h + 16) and [32 + 16h, 48 + 16h) of the 64-deep k-step (an FP8
//    operand interleaves 16-element groups, unlike FP4's one 32-run per lane
//    half); two ds_read_b128 per fragment.  The E8M0 byte of lane l still
//    scales K-block l / 32.  A row of a stage is 256 bytes = sixteen
//    16-byte chunks; logical chunk c of row r sits at c ^ (r & 15), so 16
//    consecutive rows at one chunk hit 16 different bank groups.
//  * An FP8 A stage is twice as large and a mixed FP8 x FP4 MFMA runs at the
//    FP8 rate (half the FP4 rate), so the W4A8 tile is 128 x 256: two stages
//    (64 KiB each) fit in LDS and LDS bytes per MFMA cycle equal the 256 x 256
//    FP4 kernel's.  Scale bytes are unchanged (one per 32 elements).
//
// Ragged edges: rows past M (or N) read a clamped, valid row and are never
// stored.  The copy path needs k % 512 == 0 and 16-byte aligned scale arrays;
// any other k (a multiple of 32) goes through a register path that zero-fills
// the missing 32-blocks (zero codes contribute nothing whatever their scale).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mxfp4 {
namespace {

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Chunk swizzle of a row of SHIFT = log2(16-byte chunks): rows of 8 chunks use
// (row >> 1) & 7, rows of 16 chunks row & 15.
template <int SHIFT>
__device__ __forceinline__ int row_swz(int row) {
  return SHIFT == 4 ? (row & 15) : swz(row);
}

// Tile configuration.  A8: A in FP8 E4M3 (one byte per element) with B in FP4
// (W4A8).  F8F8: both operands in FP8; a stage then covers 128 K elements, so
// each operand row of a stage is 128 bytes, as an FP4 row of a 256-K stage.
template <int BM_, int BN_, int WGM_, int WGN_, bool A8_ = false, bool F8F8_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WGM = WGM_, WGN = WGN_;               // wave grid over the tile
  static constexpr int NWAVES = WGM * WGN, THREADS = 64 * NWAVES;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr bool F8F8 = F8F8_;
  static constexpr bool A8 = A8_ || F8F8_;                   // A in FP8 E4M3 instead of FP4
  static constexpr bool B8 = F8F8_;                          // B in FP8 E4M3 instead of FP4
  static constexpr int SK = F8F8 ? 128 : 256;                // K elements per stage
  static constexpr int KSTEPS = SK / 64;                     // 64-deep MFMA k-steps per stage
  static constexpr int SB = SK / 32;                         // scale bytes per row per stage
  static constexpr int SPG_SHIFT = F8F8 ? 2 : 1;             // log2 of the stages per 16-byte scale piece
  static constexpr int A_ROW = A8 ? SK : SK / 2;             // A code bytes per row per stage
  static constexpr int B_ROW = B8 ? SK : SK / 2;             // B code bytes per row per stage
  static constexpr int A_SHIFT = A_ROW == 256 ? 4 : 3;       // log2 of the 16-byte chunks in an A row
  static constexpr int B_SHIFT = B_ROW == 256 ? 4 : 3;
  static constexpr int A_READS = A8 ? 2 : 1;                 // ds_read_b128 per A fragment
  static constexpr int B_READS = B8 ? 2 : 1;
  using AFrag = typename std::conditional<A8, v8i, v4i>::type;
  using BFrag = typename std::conditional<B8, v8i, v4i>::type;
  static constexpr int A_BYTES = BM * A_ROW, B_BYTES = BN * B_ROW;
  static constexpr int CODE_STAGE = A_BYTES + B_BYTES;
  // 16-byte scale copies per thread per group (16 scale bytes per row = two
  // stages); when BM + BN is not a multiple of the thread count the last
  // copies re-read a valid row into padding
  static constexpr int S_LOADS = (BM + BN + THREADS - 1) / THREADS;
  static constexpr int SCALE_GROUP = S_LOADS * THREADS * 16;
  static constexpr int LDS_BYTES = 2 * CODE_STAGE + 2 * SCALE_GROUP;
  static constexpr int A_LOADS = BM * A_ROW / 16 / THREADS;      // 16-byte copies per thread per stage
  static constexpr int B_LOADS = BN * B_ROW / 16 / THREADS;
  static constexpr int CODE_LOADS = A_LOADS + B_LOADS;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes");
  static_assert(BM * A_ROW % (16 * THREADS) == 0 && BN * B_ROW % (16 * THREADS) == 0,
                "code copies must split evenly over the threads");
  static_assert(!A8 || BM <= 128 || F8F8, "FP8 A: a tile's A bytes (BM * k) must stay below 2^32 for k <= 2^24");
  static_assert(WGM == 2, "the fp32 epilogue stages the tile in two halves by wave row");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tiles of whole 32x32 MFMA blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Row range of the A tile a workgroup works on (dense: [m0, min(m0+BM, M));
// grouped: the expert's rows inside this m-tile).
struct RowRange {
  int lo;     // first row of the tile
  int last;   // last valid row (reads are clamped to it)
  int end;    // one past the last row that is stored
};

// Scale layouts.  The copy path reads a row's scale bytes as 16-byte pieces,
// piece g holding the scales of the row's 32-blocks 16g .. 16g + 15 (512 K).
// Row-major scales ([rows, k/32]): piece g of row r at r * k/32 + 16 g, so the
// 64 rows of one copy instruction touch 64 cache lines.  Interleaved scales
// ([k/512, rows, 16], `scale_il`): piece g of row r at g * rows * 16 + r * 16,
// so those 64 pieces are 1 KB of consecutive bytes (8 lines).  Scale byte
// offset of a row from the tile's first row: row * scale_row_stride.
__device__ __forceinline__ uint32_t scale_row_stride(const GemmArgs& args) {
  return args.scale_il ? 16u : (uint32_t)args.k / 32;
}

// Workgroup-uniform bases of one output tile: its first A row, first B row,
// and their scale rows.  Per-thread copy offsets are taken from these, so they
// fit 32 bits (a tile spans at most 256 rows) and the bases stay in scalar
// registers.
struct TileBases {
  const uint8_t* a_q;
  const uint8_t* b_q;
  const uint8_t* a_s;
  const uint8_t* b_s;
};

template <class C>
__device__ __forceinline__ TileBases tile_bases(const GemmArgs& args, const uint8_t* b_q, const uint8_t* b_s,
                                                const RowRange& ar, int n0) {
  const int64_t ss = scale_row_stride(args), ka = C::A8 ? args.k : args.k / 2, kbb = C::B8 ? args.k : args.k / 2;
  return {args.a_q + ar.lo * ka, b_q + n0 * kbb, args.a_s + ar.lo * ss, b_s + n0 * ss};
}

// Buffer resources over the same tile operands, sized to the rows the tile
// reads (at most 256 FP4 rows or 128 FP8 rows, so at most 2^31 code bytes
// for k <= 2^24), and the byte distance between consecutive scale pieces of
// a row (row-major 16; interleaved rows * 16, at most 2^31 / (k/512)).
// Copy path only (k % 512 == 0).
struct TileRsrc {
  __amdgpu_buffer_rsrc_t a_q, b_q, a_s, b_s;
  uint32_t a_sg, b_sg;
};

template <class C>
__device__ __forceinline__ TileRsrc tile_rsrc(const TileBases& tb, const RowRange& ar, int n0, const GemmArgs& args) {
  const uint32_t k = args.k, ks = k / 32, ka = C::A8 ? k : k / 2, kbb = C::B8 ? k : k / 2;
  const uint32_t a_rows = ar.last - ar.lo + 1, b_rows = min(C::BN, args.n - n0);
  if (args.scale_il) {
    // the tile's rows in each of the k/512 slabs: the last slab's rows end the range
    const uint32_t a_sg = (uint32_t)args.m * 16, b_sg = (uint32_t)args.n * 16, last = k / 512 - 1;
    return {make_rsrc(tb.a_q, a_rows * ka), make_rsrc(tb.b_q, b_rows * kbb), make_rsrc(tb.a_s, last * a_sg + a_rows * 16),
            make_rsrc(tb.b_s, last * b_sg + b_rows * 16), a_sg, b_sg};
  }
  return {make_rsrc(tb.a_q, a_rows * ka), make_rsrc(tb.b_q, b_rows * kbb), make_rsrc(tb.a_s, a_rows * ks),
          make_rsrc(tb.b_s, b_rows * ks), 16u, 16u};
}

// Per-thread byte offsets of the copies from the tile bases, at stage 0 / scale
// group 0.  Copy j of a stage moves slot (j*NWAVES + wave)*64 + lane: row
// slot / chunks-per-row, logical 16-byte chunk (slot % chunks-per-row) ^ the
// row's swizzle.  Rows past the operand's end read its last row (never stored).
template <class C>
struct Sources {
  uint32_t a_code[C::A_LOADS];
  uint32_t b_code[C::B_LOADS];
  uint32_t scale[C::S_LOADS];    // slots below BM are A rows, the rest B rows
};

// Whether scale slot group j of wave w holds B rows: BM is a multiple of 64,
// so all 64 lanes of a wave instruction agree.
template <class C>
__device__ __forceinline__ bool scale_is_b(int j, int w) {
  return (j * C::NWAVES + w) * 64 >= C::BM;
}

template <class C>
__device__ __forceinline__ void make_sources(Sources<C>& src, const RowRange& ar, int n0, int n, int k, uint32_t ss) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t ka = C::A8 ? k : k / 2, kbb = C::B8 ? k : k / 2;
  const int a_rows = ar.last - ar.lo, b_rows = n - 1 - n0;   // largest valid row offsets
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int slot = (j * C::NWAVES + w) * 64 + lane;
    const int r = slot >> C::A_SHIFT, lc = (slot & ((1 << C::A_SHIFT) - 1)) ^ row_swz<C::A_SHIFT>(r);
    src.a_code[j] = (uint32_t)min(r, a_rows) * ka + lc * 16;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int slot = (j * C::NWAVES + w) * 64 + lane;
    const int r = slot >> C::B_SHIFT, lc = (slot & ((1 << C::B_SHIFT) - 1)) ^ row_swz<C::B_SHIFT>(r);
    src.b_code[j] = (uint32_t)min(r, b_rows) * kbb + lc * 16;
  }
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j) {
    const int slot = (j * C::NWAVES + w) * 64 + lane;
    src.scale[j] = slot >= C::BM ? (uint32_t)min(slot - C::BM, b_rows) * ss : (uint32_t)min(slot, a_rows) * ss;
  }
}

// Code copies of stage kt into `stage` (direct global -> LDS), A rows and B
// rows separately: the pipeline issues them in different k-steps.
template <class C>
__device__ __forceinline__ void copy_codes_a(uint8_t MXFP4_LDS* stage, const Sources<C>& src, const TileRsrc& tr,
                                             int kt) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: LDS base goes to M0
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j)
    buf2lds_16(tr.a_q, src.a_code[j], kt * C::A_ROW, (MXFP4_LDS void*)(stage + (j * C::NWAVES + w) * 64 * 16));
}

template <class C>
__device__ __forceinline__ void copy_codes_b(uint8_t MXFP4_LDS* stage, const Sources<C>& src, const TileRsrc& tr,
                                             int kt) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j)
    buf2lds_16(tr.b_q, src.b_code[j], kt * C::B_ROW,
               (MXFP4_LDS void*)(stage + C::A_BYTES + (j * C::NWAVES + w) * 64 * 16));
}

// Scale copies of group g (stages 2g and 2g+1): piece g of every row.
template <class C>
__device__ __forceinline__ void copy_scales(uint8_t MXFP4_LDS* group, const Sources<C>& src, const TileRsrc& tr,
                                            int g) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j)
    buf2lds_16(scale_is_b<C>(j, w) ? tr.b_s : tr.a_s, src.scale[j], g * (scale_is_b<C>(j, w) ? tr.b_sg : tr.a_sg),
               (MXFP4_LDS void*)(group + (j * C::NWAVES + w) * 64 * 16));
}

// Stage kt through registers for any k % 32 == 0: 32-blocks at or past k get
// zero codes and scale byte 127.  Writes the same LDS layout as the copies
// (the SB scale bytes of stage kt at byte SB * (kt mod stages per piece) of
// each row's 16-byte piece).
template <class C>
__device__ __forceinline__ void load_stage_generic(uint8_t MXFP4_LDS* stage, uint8_t MXFP4_LDS* group,
                                                   const Sources<C>& src, const TileBases& tb, int k, int kt) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int blocks_left = k / 32 - kt * C::SB;   // valid 32-blocks in this stage (may exceed SB)
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int slot = (j * C::NWAVES + w) * 64 + lane;
    const int lc = (slot & ((1 << C::A_SHIFT) - 1)) ^ row_swz<C::A_SHIFT>(slot >> C::A_SHIFT);
    v4i v = {0, 0, 0, 0};
    // a 32-block is one chunk of FP4 codes or two chunks of FP8 codes
    if ((lc >> (C::A8 ? 1 : 0)) < blocks_left) v = *(const v4i*)(tb.a_q + kt * C::A_ROW + src.a_code[j]);
    *(v4i MXFP4_LDS*)(stage + slot * 16) = v;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int slot = (j * C::NWAVES + w) * 64 + lane;
    const int lc = (slot & ((1 << C::B_SHIFT) - 1)) ^ row_swz<C::B_SHIFT>(slot >> C::B_SHIFT);
    v4i v = {0, 0, 0, 0};
    if ((lc >> (C::B8 ? 1 : 0)) < blocks_left) v = *(const v4i*)(tb.b_q + kt * C::B_ROW + src.b_code[j]);
    *(v4i MXFP4_LDS*)(stage + C::A_BYTES + slot * 16) = v;
  }
#pragma unroll
  for (int j = 0; j < C::S_LOADS; ++j) {
    const int slot = (j * C::NWAVES + w) * 64 + lane;
    const uint8_t* sp = (scale_is_b<C>(j, w) ? tb.b_s : tb.a_s) + kt * C::SB + src.scale[j];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      lo |= (b < blocks_left ? (uint32_t)sp[b] : 127u) << (8 * b);
      if constexpr (C::SB == 8) hi |= (b + 4 < blocks_left ? (uint32_t)sp[b + 4] : 127u) << (8 * b);
    }
    const int piece = kt & ((1 << C::SPG_SHIFT) - 1);
    if constexpr (C::SB == 8) {
      v2i word = {(int)lo, (int)hi};
      *(v2i MXFP4_LDS*)(group + slot * 16 + 8 * piece) = word;
    } else {
      *(int MXFP4_LDS*)(group + slot * 16 + 4 * piece) = (int)lo;
    }
  }
}

// Operand fragments of one 64-deep k-step for a wave's (BM/2) x (BN/2) sub-tile.
template <class C>
struct Frags {
  typename C::AFrag a[C::MI];
  typename C::BFrag b[C::NI];
};

// Scale words of one stage.  A 256-K stage has 8 scale bytes per row, two
// 32-bit words: word 0 for k-steps 0-1, word 1 for k-steps 2-3.  A 128-K stage
// (both operands FP8) has 4, one word for its two k-steps.  Lanes 32..63 feed
// the odd 32-block of each k-step, so their words are shifted right by one
// byte; k-step s then takes byte 2 * (s & 1) of word s / 2.
template <class C>
struct Scales {
  v2i a[C::MI];
  v2i b[C::NI];
};

template <class C>
__device__ __forceinline__ v2i read_scale_word(const uint8_t MXFP4_LDS* p) {
  if constexpr (C::SB == 8) {
    return *(const v2i MXFP4_LDS*)p;
  } else {
    const int w = *(const int MXFP4_LDS*)p;
    return v2i{w, w};
  }
}

// MA is the number of the wave's 32-row MFMA blocks that are computed (see
// run_tile); the others need no operands.  `piece` is the stage's index
// within its scale group (scale bytes at SB * piece of each row's 16 bytes).
template <class C, int MA = C::MI>
__device__ __forceinline__ void read_scales_raw(const uint8_t MXFP4_LDS* group, int piece, Scales<C>& sc,
                                                int wm0, int wn0, int lane) {
  if constexpr (MA > 0) {
    const uint8_t MXFP4_LDS* base = group + C::SB * piece;
#pragma unroll
    for (int i = 0; i < MA; ++i) sc.a[i] = read_scale_word<C>(base + (wm0 + 32 * i + (lane & 31)) * 16);
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
      sc.b[j] = read_scale_word<C>(base + (C::BM + wn0 + 32 * j + (lane & 31)) * 16);
  }
}

template <class C, int MA = C::MI>
__device__ __forceinline__ void shift_scales(Scales<C>& sc, int lane) {
  if constexpr (MA > 0) {
    const int shift = 8 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < MA; ++i) {
      sc.a[i].x = (int)((uint32_t)sc.a[i].x >> shift);
      sc.a[i].y = (int)((uint32_t)sc.a[i].y >> shift);
    }
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      sc.b[j].x = (int)((uint32_t)sc.b[j].x >> shift);
      sc.b[j].y = (int)((uint32_t)sc.b[j].y >> shift);
    }
  }
}

// One operand fragment of k-step S of row r from a stage row of ROW bytes.
// An FP4 operand: lane half h holds the 32 elements K [32h, 32h + 32) of the
// k-step, chunk 2S + h.  An FP8 operand interleaves 16-element groups: lane
// half h holds K [16h, 16h + 16) of the k-step in its first four registers and
// [32 + 16h, 48 + 16h) in the last four (measured through the library with
// one-hot rows), i.e. chunks 4S + h and 4S + 2 + h.
template <bool FP8, int ROW, int SHIFT, int S>
__device__ __forceinline__ typename std::conditional<FP8, v8i, v4i>::type read_frag(
    const uint8_t MXFP4_LDS* rows, int r, int lane) {
  const int h = lane >> 5;
  const uint8_t MXFP4_LDS* row = rows + r * ROW;
  if constexpr (FP8) {
    const v4i lo = *(const v4i MXFP4_LDS*)(row + (((4 * S + h) ^ row_swz<SHIFT>(r)) << 4));
    const v4i hi = *(const v4i MXFP4_LDS*)(row + (((4 * S + 2 + h) ^ row_swz<SHIFT>(r)) << 4));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  } else {
    return *(const v4i MXFP4_LDS*)(row + (((2 * S + h) ^ row_swz<SHIFT>(r)) << 4));
  }
}

template <class C, int S, int MA = C::MI>
__device__ __forceinline__ void read_frags(const uint8_t MXFP4_LDS* stage, Frags<C>& f, int wm0, int wn0,
                                           int lane) {
  if constexpr (MA > 0) {
#pragma unroll
    for (int i = 0; i < MA; ++i)
      f.a[i] = read_frag<C::A8, C::A_ROW, C::A_SHIFT, S>(stage, wm0 + 32 * i + (lane & 31), lane);
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
      f.b[j] = read_frag<C::B8, C::B_ROW, C::B_SHIFT, S>(stage + C::A_BYTES, wn0 + 32 * j + (lane & 31), lane);
  }
}

// MFMAs of k-step S over the MFMA blocks [I0, I1) x [0, NI).
template <class C, int S, int I0, int I1>
__device__ __forceinline__ void mma_kstep(const Frags<C>& f, const Scales<C>& sc, v16f (&acc)[C::MI][C::NI]) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      const int sa = (S < 2) ? sc.a[i].x : sc.a[i].y;
      const int sb = (S < 2) ? sc.b[j].x : sc.b[j].y;
      if constexpr (C::F8F8)
        acc[i][j] = mfma32_fp8<2 * (S & 1)>(f.b[j], f.a[i], acc[i][j], sb, sa);
      else if constexpr (C::A8)
        acc[i][j] = mfma32_fp4_fp8<2 * (S & 1)>(f.b[j], f.a[i], acc[i][j], sb, sa);
      else
        acc[i][j] = mfma32_fp4<2 * (S & 1)>(f.b[j], f.a[i], acc[i][j], sb, sa);
    }
}

// Workgroup barrier without a memory fence: copies into LDS are tracked with
// explicit vmcnt waits, so the fence of __syncthreads() (which would also wait
// for the copies still streaming in) is not wanted.  The asm memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  MXFP4_WAIT_LGKM0();
  asm volatile("s_barrier" ::: "memory");
}

// Epilogue.  Each wave converts its accumulators and writes them into a
// row-major tile in LDS (rows padded by 16 bytes so the 32 rows a wave writes
// at one column spread over the banks); then all 256 threads copy the tile out
// in 16-byte row-contiguous pieces, so global stores are fully coalesced and
// the code stays small (edge guards live in one loop, not in every unrolled
// store).  BF16 uses the hardware packed convert (nearest-even).  The fp32
// tile does not fit in LDS at once and goes out in two halves by wave row.
// The caller must have ended every LDS read and copy of the main loop.
template <class C, int ESIZE, int PITCH, int SWZ_MASK = 0>
__device__ __forceinline__ void copy_out(const GemmArgs& args, const uint8_t MXFP4_LDS* tile, int row_begin,
                                         int rows, const RowRange& ar, int n0) {
  constexpr int esize = ESIZE;
  constexpr int CPR = C::BN * ESIZE / 16;                  // 16-byte chunks per tile row (power of two)
  const int n = args.n;
  const int valid_rows = min(rows, ar.end - ar.lo - row_begin);
  const int valid_cols = min(C::BN, n - n0);
  const bool vec_ok = ((n * ESIZE) & 15) == 0;
  uint8_t* cbase = (uint8_t*)args.c + ((int64_t)(ar.lo + row_begin) * n + n0) * ESIZE;
  const int64_t row_bytes = (int64_t)n * ESIZE;
  for (int idx = threadIdx.x; idx < valid_rows * CPR; idx += C::THREADS) {
    const int r = idx / CPR, cc = idx % CPR;
    const int col = cc * (16 / ESIZE);
    if (col >= valid_cols) continue;
    const v4i v = *(const v4i MXFP4_LDS*)(tile + r * PITCH + ((cc ^ (r & SWZ_MASK)) * 16));
    uint8_t* dst = cbase + r * row_bytes + cc * 16;
    const int cnt = min(16 / ESIZE, valid_cols - col);
    if (vec_ok && cnt * ESIZE == 16) {
      // non-temporal: C is not re-read here, and lines that bypass the L2
      // leave less to write back when the kernel ends (measured 3-4 % faster)
      __builtin_nontemporal_store(v, (v4i*)dst);
    } else if (esize == 4) {
      for (int e = 0; e < cnt; ++e) ((uint32_t*)dst)[e] = (uint32_t)(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
    } else {
      for (int e = 0; e < cnt; ++e) {
        const uint32_t word = (uint32_t)((e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w);
        ((uint16_t*)dst)[e] = (uint16_t)(word >> (16 * (e & 1)));
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void store_tile(const GemmArgs& args, const v16f (&acc)[C::MI][C::NI],
                                           const RowRange& ar, int n0, int wm0, int wn0, int lane,
                                           uint8_t MXFP4_LDS* lds) {
  if (!args.c_f32) {
    constexpr int PITCH = C::BN * 2 + 16;
    static_assert(C::BM * PITCH <= C::LDS_BYTES, "bf16 tile must fit in the pipeline LDS");
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm0 + 32 * i + (lane & 31);
          const int col = wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
          bf16x2_t lo = {(__bf16)acc[i][j][4 * q + 0], (__bf16)acc[i][j][4 * q + 1]};
          bf16x2_t hi = {(__bf16)acc[i][j][4 * q + 2], (__bf16)acc[i][j][4 * q + 3]};
          v2i pk = {__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
          *(v2i MXFP4_LDS*)(lds + r * PITCH + col * 2) = pk;
        }
    __syncthreads();
    copy_out<C, 2, PITCH>(args, lds, 0, C::BM, ar, n0);
  } else {
    constexpr int PITCH = C::BN * 4 + 16;
    static_assert(C::WM * PITCH <= C::LDS_BYTES, "fp32 half tile must fit in the pipeline LDS");
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm0 == half * C::WM) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 32 * i + (lane & 31);
              const int col = wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
              v4f val = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              *(v4f MXFP4_LDS*)(lds + r * PITCH + col * 4) = val;
            }
      }
      __syncthreads();
      copy_out<C, 4, PITCH>(args, lds, half * C::WM, C::WM, ar, n0);
      __syncthreads();
    }
  }
}

// Scheduling pattern for one k-step's MFMAs: READS fragment reads for the next
// k-step go out one per MFMA over the first MFMAs, and COPIES global -> LDS
// copies are spread evenly over all of them.  A burst of reads or copies would
// stall the wave at issue (full LDS or vector-memory queue) while its MFMAs
// wait behind it; spread out, they drain while the MFMAs run.
// sched_barrier(0) closes the region.
template <int READS, int COPIES, int MFMAS, int I>
__device__ __forceinline__ void kstep_slots() {
  if constexpr (I < MFMAS) {
    if constexpr (I < READS) __builtin_amdgcn_sched_group_barrier(0x100, I + 1 < MFMAS ? 1 : READS - I, 0);
    constexpr int copies = COPIES * (I + 1) / MFMAS - COPIES * I / MFMAS;
    if constexpr (copies > 0) __builtin_amdgcn_sched_group_barrier(0x020, copies, 0);   // VMEM copies
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  // MFMA
    kstep_slots<READS, COPIES, MFMAS, I + 1>();
  }
}

template <class C, int COPIES, int MA = C::MI>
__device__ __forceinline__ void kstep_pattern() {
  kstep_slots<(MA > 0 ? MA * C::A_READS + C::NI * C::B_READS : 0), COPIES, MA * C::NI, 0>();
  __builtin_amdgcn_sched_barrier(0);
}

// One pipelined stage (straight-line code: every branch is a template
// parameter, so the compiler cannot sink the MFMAs past the barrier).
// On entry fa holds k-step 0 of stage kt and sc its scales; on exit, if NEXT,
// fa/sc hold k-step 0 of stage kt+1.  COPY_CODES / COPY_SCALES issue the copies
// of stage kt+2 (and of its scale group) once stage kt's buffer is released,
// spread over the MFMAs of the last k-step.
// The copies a stage issues (COPY_CODES / COPY_SCALES): stage `stage` and scale
// group `group` of the tile that `src` / `tr` describe, into the code buffer this
// stage releases and scale buffer `group_buf`.  In the main loop that is the
// same tile's stage kt + 2; in the persistent loop's last stages, the next
// tile's stage 0 and scale group 0.
struct StageCopy {
  int stage, group, group_buf;
};

template <class C, int MA, bool NEXT, bool COPY_CODES, bool COPY_SCALES>
__device__ __forceinline__ void pipelined_stage_from(v16f (&acc)[C::MI][C::NI], Frags<C>& fa, Frags<C>& fb,
                                                     Scales<C>& sc, const Sources<C>& src, const TileRsrc& tr,
                                                     const StageCopy& cp, uint8_t MXFP4_LDS* lds, int kt, int wm0,
                                                     int wn0, int lane) {
  constexpr int L = C::KSTEPS - 1;   // the last k-step; its fragments arrive in fb
  constexpr int G = C::SPG_SHIFT;    // stages per scale group: 1 << G
  uint8_t MXFP4_LDS* cur = lds + (kt & 1) * C::CODE_STAGE;
  uint8_t MXFP4_LDS* nxt = lds + ((kt + 1) & 1) * C::CODE_STAGE;
  // Fragment reads run one k-step ahead of the MFMAs.  Before a new batch of
  // reads is issued, the previous batch (issued a whole k-step earlier, so
  // already landed) is retired with lgkmcnt(0): the LDS counter holds at most
  // 15 operations, and with two batches pending the compiler could only wait
  // for both, stalling on the batch just issued.
  read_frags<C, 1, MA>(cur, fb, wm0, wn0, lane);
  mma_kstep<C, 0, 0, MA>(fa, sc, acc);
  kstep_pattern<C, 0, MA>();
  if constexpr (C::KSTEPS == 4) {
    MXFP4_WAIT_LGKM0();
    read_frags<C, 2, MA>(cur, fa, wm0, wn0, lane);
    mma_kstep<C, 1, 0, MA>(fb, sc, acc);
    kstep_pattern<C, 0, MA>();
    MXFP4_WAIT_LGKM0();
    read_frags<C, 3, MA>(cur, fb, wm0, wn0, lane);
    mma_kstep<C, 2, 0, MA>(fa, sc, acc);
    kstep_pattern<C, 0, MA>();
  }
  if (NEXT) {
    // stage kt+1 and its scales have landed; stage kt is fully read once every
    // wave has passed the barrier
    MXFP4_WAIT_VMCNT(0);
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    read_frags<C, 0, MA>(nxt, fa, wm0, wn0, lane);
    if (COPY_SCALES) copy_scales<C>(lds + 2 * C::CODE_STAGE + cp.group_buf * C::SCALE_GROUP, src, tr, cp.group);
    if (COPY_CODES) {
      copy_codes_a<C>(cur, src, tr, cp.stage);
      copy_codes_b<C>(cur, src, tr, cp.stage);
    }
    mma_kstep<C, L, 0, MA>(fb, sc, acc);
    // the next stage's first fragments go out before the copies (measured ~2 %
    // faster than interleaving them one per MFMA)
    if constexpr (MA > 0) __builtin_amdgcn_sched_group_barrier(0x100, MA * C::A_READS + C::NI * C::B_READS, 0);
    kstep_slots<0, (COPY_CODES ? C::CODE_LOADS : 0) + (COPY_SCALES ? C::S_LOADS : 0), MA * C::NI, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // the next stage's scale words replace this stage's once its last MFMAs are issued
    read_scales_raw<C, MA>(lds + 2 * C::CODE_STAGE + (((kt + 1) >> G) & 1) * C::SCALE_GROUP,
                           (kt + 1) & ((1 << G) - 1), sc, wm0, wn0, lane);
    shift_scales<C, MA>(sc, lane);
  } else {
    MXFP4_WAIT_LGKM0();
    mma_kstep<C, L, 0, MA>(fb, sc, acc);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// A stage of the main loop: its copies are the same tile's stage kt + 2.
template <class C, int MA, bool NEXT, bool COPY_CODES, bool COPY_SCALES>
__device__ __forceinline__ void pipelined_stage(v16f (&acc)[C::MI][C::NI], Frags<C>& fa, Frags<C>& fb,
                                                Scales<C>& sc, const Sources<C>& src, const TileRsrc& tr,
                                                uint8_t MXFP4_LDS* lds, int kt, int wm0, int wn0, int lane) {
  constexpr int G = C::SPG_SHIFT;
  const StageCopy cp{kt + 2, (kt + 2) >> G, ((kt + 2) >> G) & 1};
  pipelined_stage_from<C, MA, NEXT, COPY_CODES, COPY_SCALES>(acc, fa, fb, sc, src, tr, cp, lds, kt, wm0, wn0, lane);
}

// Stages kt + J .. kt + SPG - 1 of one scale group's worth of stages (SPG =
// stages per scale group).  In the loop body (TAIL false) stage kt + J copies
// stage kt + J + 2, and the stage whose copies start a new scale group (J =
// SPG - 2) also copies that group.  In the tail (the last SPG stages) only
// stages before the last two copy, and the last stage has no successor.
template <class C, int MA, int J, bool TAIL>
__device__ __forceinline__ void group_stages(v16f (&acc)[C::MI][C::NI], Frags<C>& fa, Frags<C>& fb, Scales<C>& sc,
                                             const Sources<C>& src, const TileRsrc& tr, uint8_t MXFP4_LDS* lds,
                                             int kt, int wm0, int wn0, int lane) {
  constexpr int SPG = 1 << C::SPG_SHIFT;
  if constexpr (J < SPG) {
    if constexpr (!TAIL)
      pipelined_stage<C, MA, true, true, J == SPG - 2>(acc, fa, fb, sc, src, tr, lds, kt + J, wm0, wn0, lane);
    else
      pipelined_stage<C, MA, (J < SPG - 1), (J < SPG - 2), false>(acc, fa, fb, sc, src, tr, lds, kt + J, wm0,
                                                                   wn0, lane);
    group_stages<C, MA, J + 1, TAIL>(acc, fa, fb, sc, src, tr, lds, kt, wm0, wn0, lane);
  }
}

// Main loop of the copy path with MA computed row blocks per wave.  nk = k /
// SK stages, a multiple of the stages per scale group (k % 512 == 0).
template <class C, int MA>
__device__ __forceinline__ void copy_loop(v16f (&acc)[C::MI][C::NI], const Sources<C>& src, const TileRsrc& tr,
                                          uint8_t MXFP4_LDS* lds, int nk, int wm0, int wn0, int lane) {
  constexpr int SPG = 1 << C::SPG_SHIFT;
  uint8_t MXFP4_LDS* group0 = lds + 2 * C::CODE_STAGE;
  copy_scales<C>(group0, src, tr, 0);
  copy_codes_a<C>(lds, src, tr, 0);
  copy_codes_b<C>(lds, src, tr, 0);
  copy_codes_a<C>(lds + C::CODE_STAGE, src, tr, 1);
  copy_codes_b<C>(lds + C::CODE_STAGE, src, tr, 1);
  MXFP4_WAIT_VMCNT(C::CODE_LOADS);            // scales and stage 0 have landed
  barrier_lds();
  Scales<C> sc;
  Frags<C> fa, fb;
  read_scales_raw<C, MA>(group0, 0, sc, wm0, wn0, lane);
  read_frags<C, 0, MA>(lds, fa, wm0, wn0, lane);
  shift_scales<C, MA>(sc, lane);
  int kt = 0;
  for (; kt + SPG < nk; kt += SPG) group_stages<C, MA, 0, false>(acc, fa, fb, sc, src, tr, lds, kt, wm0, wn0, lane);
  group_stages<C, MA, 0, true>(acc, fa, fb, sc, src, tr, lds, kt, wm0, wn0, lane);
}

// copy_loop<C, active> and then the epilogue `epi` for a wave-uniform active
// in [0, C::MI].  The epilogue runs inside each branch: with the branches
// merged before it, the accumulators of every branch meet in one set of
// registers, and with 256 accumulators per wave (one wave per SIMD) the
// register allocator moved all of them out of the accumulator registers at
// once and spilled.
template <class C, int MA, class Epi>
__device__ __forceinline__ void copy_loop_dispatch(int active, v16f (&acc)[C::MI][C::NI], const Sources<C>& src,
                                                   const TileRsrc& tr, uint8_t MXFP4_LDS* lds, int nk, int wm0,
                                                   int wn0, int lane, const Epi& epi) {
  if constexpr (MA == 0) {
    copy_loop<C, 0>(acc, src, tr, lds, nk, wm0, wn0, lane);
    epi(acc);
  } else {
    if (active >= MA) {
      copy_loop<C, MA>(acc, src, tr, lds, nk, wm0, wn0, lane);
      epi(acc);
    } else {
      copy_loop_dispatch<C, MA - 1>(active, acc, src, tr, lds, nk, wm0, wn0, lane, epi);
    }
  }
}

// Main loop + epilogue for one output tile.
template <class C, bool COPY>
__device__ __forceinline__ void run_tile(const GemmArgs& args, const uint8_t* b_q, const uint8_t* b_s,
                                         const RowRange& ar, int n0, uint8_t MXFP4_LDS* lds) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Wave w runs on SIMD w % 4.  With 8 waves, the two waves sharing a SIMD sit
  // in different wave rows: in a tile whose last rows are padding, the work
  // the second wave row skips (copy_loop_dispatch) is spread over all SIMDs
  // instead of idling two of them.
  const int wm0 = (w / C::WGN) * C::WM, wn0 = (w % C::WGN) * C::WN;
  v16f acc[C::MI][C::NI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Sources<C> src;
  make_sources<C>(src, ar, n0, args.n, args.k, scale_row_stride(args));
  const TileBases tb = tile_bases<C>(args, b_q, b_s, ar, n0);
  uint8_t MXFP4_LDS* group0 = lds + 2 * C::CODE_STAGE;

  const auto epi = [&](v16f (&a)[C::MI][C::NI]) {
    MXFP4_WAIT_VMCNT(0);
    __syncthreads();   // every wave is done with the pipeline buffers
    store_tile<C>(args, a, ar, n0, wm0, wn0, lane, lds);
  };
  if (COPY) {
    // Row blocks of 32 that lie wholly past the tile's last stored row (the
    // tail of an expert's rows, or of a ragged M) need no MFMAs or operand
    // reads; their accumulators stay zero and are never stored.  Every wave
    // still issues all copies and meets every barrier.
    const int active = __builtin_amdgcn_readfirstlane(min(max((ar.end - ar.lo - wm0 + 31) / 32, 0), C::MI));
    const TileRsrc tr = tile_rsrc<C>(tb, ar, n0, args);
    copy_loop_dispatch<C, C::MI>(active, acc, src, tr, lds, args.k / C::SK, wm0, wn0, lane, epi);
  } else {
    const int nk = (args.k + C::SK - 1) / C::SK;
    for (int kt = 0; kt < nk; ++kt) {
      load_stage_generic<C>(lds, group0, src, tb, args.k, kt);
      __syncthreads();
      Scales<C> sc;
      Frags<C> f;
      read_scales_raw<C>(group0, kt & ((1 << C::SPG_SHIFT) - 1), sc, wm0, wn0, lane);
      shift_scales<C>(sc, lane);
      read_frags<C, 0>(lds, f, wm0, wn0, lane);
      mma_kstep<C, 0, 0, C::MI>(f, sc, acc);
      read_frags<C, 1>(lds, f, wm0, wn0, lane);
      mma_kstep<C, 1, 0, C::MI>(f, sc, acc);
      if constexpr (C::KSTEPS == 4) {
        read_frags<C, 2>(lds, f, wm0, wn0, lane);
        mma_kstep<C, 2, 0, C::MI>(f, sc, acc);
        read_frags<C, 3>(lds, f, wm0, wn0, lane);
        mma_kstep<C, 3, 0, C::MI>(f, sc, acc);
      }
      __syncthreads();
    }
    epi(acc);
  }
}

template <class C, bool COPY>
__global__ __launch_bounds__(C::THREADS) void gemm_tile_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
  RowRange ar;
  ar.lo = tm * C::BM;
  ar.end = min(ar.lo + C::BM, args.m);
  ar.last = ar.end - 1;
  run_tile<C, COPY>(args, args.b_q, args.b_s, ar, tn * C::BN, (uint8_t MXFP4_LDS*)smem);
}

// Rows [lo, hi) of group g = base + lane within one chunk of 64 groups.  Each
// offset is clamped into [0, total_m] and replaced by the running maximum of
// the clamped offsets before it (`carry` holds it from the previous chunk), so
// any offsets give non-decreasing, disjoint, in-range segments: hi of group g is
// lo of group g + 1, the segments cover at most total_m rows in all, and their
// m-tiles number at most ceil(total_m / bm) + groups (the grid's bound).  For
// valid offsets (non-decreasing, 0 .. total_m) the segments are the offsets'.
// Lanes past the last group get an empty segment.  Returns the chunk's last hi
// (wave-uniform), the carry of the next chunk.
__device__ __forceinline__ int chunk_rows(const int32_t* offsets, int groups, int total_m, int base, int carry,
                                          int& lo, int& hi) {
  const int lane = threadIdx.x & 63;
  const int g = base + lane;
  const bool valid = g < groups;
  const int c = valid ? min(max(offsets[g], 0), total_m) : 0;
  const int e = valid ? min(max(offsets[g + 1], 0), total_m) : 0;
  int pm = c;   // inclusive running maximum of the chunk's clamped start offsets
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(pm, d, 64);
    if (lane >= d) pm = max(pm, o);
  }
  lo = max(pm, carry);
  hi = max(lo, e);
  if (!valid) hi = lo;
  const int last = min(63, groups - 1 - base);
  return __builtin_amdgcn_readfirstlane(__shfl(hi, last, 64));
}

// Number of m-tiles over all groups, ceil(rows_g / bm) each (wave-uniform).
__device__ __forceinline__ int count_mtiles(const int32_t* offsets, int groups, int total_m, int bm) {
  int cnt = 0, carry = 0;
  for (int base = 0; base < groups; base += 64) {
    int lo, hi;
    carry = chunk_rows(offsets, groups, total_m, base, carry, lo, hi);
    cnt += (hi - lo + bm - 1) / bm;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d, 64);
  return __builtin_amdgcn_readfirstlane(cnt);   // uniform: keep it (and what follows) in scalar registers
}

// An expert's share of the m-tiles: m-tiles [first, first + cnt) over its
// sanitized rows [lo, hi).
struct ExpertTiles {
  int g, first, cnt, lo, hi;
};

// Finds the expert owning global m-tile `mt` (m-tiles are counted expert by
// expert, ceil(rows_g / BM) per expert, over the segments of chunk_rows).
__device__ __forceinline__ bool find_expert(const int32_t* offsets, int groups, int total_m, int bm, int mt,
                                            ExpertTiles& e) {
  const int lane = threadIdx.x & 63;
  int carry = 0, carry_rows = 0;
  for (int base = 0; base < groups; base += 64) {
    const int g = base + lane;
    int lo, hi;
    carry_rows = chunk_rows(offsets, groups, total_m, base, carry_rows, lo, hi);
    const int cnt = (hi - lo + bm - 1) / bm;
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
      // every value below is wave-uniform; readfirstlane puts it in scalar
      // registers, so the expert's operand buffer resources are scalar too
      // (a per-lane resource wraps every copy in a waterfall loop: measured
      // 10 % slower on the MoE layer)
      const int src = __ffsll((long long)mask) - 1;
      e.g = __builtin_amdgcn_readfirstlane(__shfl(g, src, 64));
      e.lo = __builtin_amdgcn_readfirstlane(__shfl(lo, src, 64));
      e.hi = __builtin_amdgcn_readfirstlane(__shfl(hi, src, 64));
      e.cnt = __builtin_amdgcn_readfirstlane(__shfl(cnt, src, 64));
      e.first = carry + __builtin_amdgcn_readfirstlane(__shfl(excl, src, 64));
      return true;
    }
    carry += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  }
  return false;
}

// Tile `local` of an expert with `cnt` m-tiles: the expert's m-tiles go in
// groups of four, and inside a group the m-tile runs fastest, then the
// n-tile.  Consecutive tiles (dealt to neighbouring workgroups of one XCD in
// the same round) then share a weight panel across the group's m-tiles and an
// A panel across the n-tiles a round covers: about 4 A panels and 8 weight
// panels per 32 tiles.  Plain n-tile-major order (the same thing for experts
// of at most four m-tiles) reads the A panels of all of a large expert's
// m-tiles in every round: MoE layer 255.5-256.1 -> 251.3-252.2 us on one box
// (groups of two 252.5-253.8, of eight 252.1-254.1).
__device__ __forceinline__ void expert_tile(int local, int cnt, int tiles_n, int& tn, int& mi) {
  constexpr int GM = 4;
  const int grp = local / (GM * tiles_n);
  const int rest = local - grp * GM * tiles_n;
  const int gm = min(GM, cnt - grp * GM);   // the last group may hold fewer m-tiles
  tn = rest / gm;
  mi = grp * GM + rest - tn * gm;
}

// The grid is a multiple of 8 workgroups covering at least every possible
// m-tile (the host cannot see the device offsets).  Workgroups are dispatched
// to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8; the real tiles
// are split evenly over the XCDs as contiguous ranges (consecutive tiles of one
// expert share that XCD's L2), and the spare workgroups of every XCD exit.
// Inside an expert the tiles run in the order of expert_tile, as in the
// persistent kernel (n-tile-major, its special case for small experts: W4A8
// MoE layer 412 -> 407 us on one box against m-tile-major).
template <class C, bool COPY>
__global__ __launch_bounds__(C::THREADS) void grouped_tile_kernel(GemmArgs args, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int total = count_mtiles(args.offsets, args.groups, args.m, C::BM) * tiles_n;
  const int share = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * share + slot;
  if (slot >= share || t >= total) return;
  ExpertTiles e;
  if (!find_expert(args.offsets, args.groups, args.m, C::BM, t / tiles_n, e)) return;
  const int local = t - e.first * tiles_n;   // in [0, cnt * tiles_n)
  int tn, mi;
  expert_tile(local, e.cnt, tiles_n, tn, mi);
  RowRange ar;
  ar.lo = e.lo + mi * C::BM;
  ar.end = min(e.hi, ar.lo + C::BM);
  ar.last = ar.end - 1;
  const int g = e.g;
  const int64_t kb = C::B8 ? args.k : args.k / 2, ks = args.k / 32;
  const uint8_t* b_q = args.b_q + (int64_t)g * args.n * kb;
  const uint8_t* b_s = args.b_s + (int64_t)g * args.n * ks;
  run_tile<C, COPY>(args, b_q, b_s, ar, tn * C::BN, (uint8_t MXFP4_LDS*)smem);
}

// ---------------------------------------------------------------------------
// Persistent tile loop.  One workgroup per compute unit loops over its share
// of the output tiles.  While its last stage of a tile runs, it already copies
// the next tile's first stage and scale group into the LDS that the tile no
// longer needs, and it stages the tile's epilogue through the last stage's
// buffer alone, so the next tile's first data is in flight during the
// epilogue instead of after it (a new workgroup would start from nothing).
// Needs k % (512 * 2) == 0 for FP4 (an even number of scale groups per tile,
// so every tile's scale group 0 lands in scale buffer 0).

// The wave-uniform description of one output tile.
struct TileJob {
  RowRange ar;
  int n0;
  const uint8_t* b_q;   // the B operand of the tile's group (dense: args.b_q)
  const uint8_t* b_s;
};

template <class C>
__device__ __forceinline__ void job_sources(const GemmArgs& args, const TileJob& jb, Sources<C>& src, TileRsrc& tr) {
  make_sources<C>(src, jb.ar, jb.n0, args.n, args.k, scale_row_stride(args));
  const TileBases tb = tile_bases<C>(args, jb.b_q, jb.b_s, jb.ar, jb.n0);
  tr = tile_rsrc<C>(tb, jb.ar, jb.n0, args);
}

// Epilogue through one 64 KiB region (the LDS buffer of the tile's last
// stage).  256 x 256 tiles: BF16 in two passes of 128 rows (one wave row
// each), fp32 in four passes of 64 rows.  128 x 256 tiles (W4A8): BF16 in one
// pass of both wave rows, fp32 in two passes of 64 rows (one wave row each).
// Rows are not padded: 16-byte chunk c of row r sits at chunk
// c ^ (r mod chunks-per-row), so the 32 rows one wave writes at one column
// fall in different chunks.  Ends with a barrier: the region is free.
template <class C>
__device__ __forceinline__ void store_tile_region(const GemmArgs& args, const v16f (&acc)[C::MI][C::NI],
                                                  const RowRange& ar, int n0, int wm0, int wn0, int lane,
                                                  uint8_t MXFP4_LDS* region) {
  static_assert(C::BN == 256 && ((C::BM == 256 && C::WM == 128) || (C::BM == 128 && C::WM == 64)),
                "the split epilogue is laid out for 256 x 256 and 128 x 256 tiles");
  // The LDS addresses below are the same for every tile; computed from a lane
  // index the compiler cannot see through, they are not hoisted out of the
  // persistent loop (held across the main loop they overflowed the registers).
  asm volatile("" : "+v"(lane));
  if (!args.c_f32) {
    constexpr int PITCH = C::BN * 2, CHUNKS = PITCH / 16;   // 512 bytes, 32 chunks per row
    constexpr int RP = 65536 / PITCH;                        // 128 rows per pass
#pragma unroll
    for (int pass = 0; pass < C::BM / RP; ++pass) {
      if (C::BM == RP || wm0 == pass * C::WM) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = (C::BM == RP ? wm0 : 0) + 32 * i + (lane & 31);
              const int col = wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
              bf16x2_t lo = {(__bf16)acc[i][j][4 * q + 0], (__bf16)acc[i][j][4 * q + 1]};
              bf16x2_t hi = {(__bf16)acc[i][j][4 * q + 2], (__bf16)acc[i][j][4 * q + 3]};
              v2i pk = {__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
              *(v2i MXFP4_LDS*)(region + r * PITCH + (((col >> 3) ^ (r & (CHUNKS - 1))) << 4) + (col & 7) * 2) = pk;
            }
      }
      __syncthreads();
      copy_out<C, 2, PITCH, CHUNKS - 1>(args, region, pass * RP, RP, ar, n0);
      __syncthreads();
    }
  } else {
    constexpr int PITCH = C::BN * 4, CHUNKS = PITCH / 16;   // 1024 bytes, 64 chunks per row
    constexpr int PASSES_PER_ROW = C::WM / 64;               // 64-row passes per wave row
#pragma unroll
    for (int pass = 0; pass < C::BM / 64; ++pass) {
      if (wm0 == (pass / PASSES_PER_ROW) * C::WM) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (pass % PASSES_PER_ROW) + ii;
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r = 32 * ii + (lane & 31);
              const int col = wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
              v4f val = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              *(v4f MXFP4_LDS*)(region + r * PITCH + (((col >> 2) ^ (r & (CHUNKS - 1))) << 4)) = val;
            }
        }
      }
      __syncthreads();
      copy_out<C, 4, PITCH, CHUNKS - 1>(args, region, pass * 64, 64, ar, n0);
      __syncthreads();
    }
  }
}

// One tile of the persistent loop with MA computed row blocks per wave.  On
// entry the tile's scale group 0 and stage 0 have been issued (or have landed)
// and its stage 1 is in flight; `src` / `tr` describe the tile.  `next` is the
// tile that follows (or this one again when none does): its scale group 0 and
// stage 0 are copied during this tile's last two stages, and on return `src` /
// `tr` describe it.
template <class C, int MA>
__device__ __forceinline__ void persistent_tile(const GemmArgs& args, const TileJob& cur, const TileJob& next,
                                                v16f (&acc)[C::MI][C::NI], Sources<C>& src, TileRsrc& tr,
                                                uint8_t MXFP4_LDS* lds, int nk, int wm0, int wn0, int lane) {
  constexpr int G = C::SPG_SHIFT;
  static_assert(G == 1, "the persistent loop is written for two stages per scale group");
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  uint8_t MXFP4_LDS* group0 = lds + 2 * C::CODE_STAGE;
  MXFP4_WAIT_VMCNT(C::CODE_LOADS);            // scale group 0 and stage 0 have landed
  barrier_lds();
  Scales<C> sc;
  Frags<C> fa, fb;
  read_scales_raw<C, MA>(group0, 0, sc, wm0, wn0, lane);
  read_frags<C, 0, MA>(lds, fa, wm0, wn0, lane);
  shift_scales<C, MA>(sc, lane);
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) group_stages<C, MA, 0, false>(acc, fa, fb, sc, src, tr, lds, kt, wm0, wn0, lane);
  // stage nk - 2 releases buffer 0 and scale buffer 0 (nk / 2 groups, an even
  // number): the next tile's stage 0 and scale group 0 go there
  job_sources<C>(args, next, src, tr);
  const StageCopy first{0, 0, 0};
  pipelined_stage_from<C, MA, true, true, true>(acc, fa, fb, sc, src, tr, first, lds, kt, wm0, wn0, lane);
  pipelined_stage<C, MA, false, false, false>(acc, fa, fb, sc, src, tr, lds, kt + 1, wm0, wn0, lane);
  barrier_lds();   // every wave is done with stage nk - 1's buffer, the epilogue's region
  store_tile_region<C>(args, acc, cur.ar, cur.n0, wm0, wn0, lane, lds + C::CODE_STAGE);
}

template <class C, int MA>
__device__ __forceinline__ void persistent_tile_dispatch(int active, const GemmArgs& args, const TileJob& cur,
                                                         const TileJob& next, v16f (&acc)[C::MI][C::NI],
                                                         Sources<C>& src, TileRsrc& tr, uint8_t MXFP4_LDS* lds,
                                                         int nk, int wm0, int wn0, int lane) {
  if constexpr (MA == 0) {
    persistent_tile<C, 0>(args, cur, next, acc, src, tr, lds, nk, wm0, wn0, lane);
  } else {
    if (active >= MA)
      persistent_tile<C, MA>(args, cur, next, acc, src, tr, lds, nk, wm0, wn0, lane);
    else
      persistent_tile_dispatch<C, MA - 1>(active, args, cur, next, acc, src, tr, lds, nk, wm0, wn0, lane);
  }
}

// The loop over the tiles t = first, first + step, ... < end; job(t) gives a
// tile's description.
template <class C, class JobOf>
__device__ __forceinline__ void persistent_loop(const GemmArgs& args, int first, int step, int end, const JobOf& job_of,
                                                uint8_t MXFP4_LDS* lds) {
  if (first >= end) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm0 = (w / C::WGN) * C::WM, wn0 = (w % C::WGN) * C::WN;
  const int nk = args.k / C::SK;
  v16f acc[C::MI][C::NI];
  Sources<C> src;
  TileRsrc tr;
  TileJob cur = job_of(first);
  job_sources<C>(args, cur, src, tr);
  copy_scales<C>(lds + 2 * C::CODE_STAGE, src, tr, 0);
  copy_codes_a<C>(lds, src, tr, 0);
  copy_codes_b<C>(lds, src, tr, 0);
  copy_codes_a<C>(lds + C::CODE_STAGE, src, tr, 1);
  copy_codes_b<C>(lds + C::CODE_STAGE, src, tr, 1);
  for (int t = first;;) {
    const int tn = t + step;
    const bool has_next = tn < end;
    // without a next tile the last stages re-copy this tile's first stage
    // (read, never used) so that every path issues the same copies
    const TileJob next = has_next ? job_of(tn) : cur;
    const int active = __builtin_amdgcn_readfirstlane(min(max((cur.ar.end - cur.ar.lo - wm0 + 31) / 32, 0), C::MI));
    persistent_tile_dispatch<C, C::MI>(active, args, cur, next, acc, src, tr, lds, nk, wm0, wn0, lane);
    if (!has_next) break;
    // the epilogue has freed buffer 1: the next tile's stage 1 goes there
    copy_codes_a<C>(lds + C::CODE_STAGE, src, tr, 1);
    copy_codes_b<C>(lds + C::CODE_STAGE, src, tr, 1);
    cur = next;
    t = tn;
  }
  MXFP4_WAIT_VMCNT(0);   // the last re-copy lands before the workgroup's LDS is released
}

// Dense persistent kernel: grid = a multiple of 8 workgroups, at most one per
// CU; workgroup b runs on XCD b % 8 and takes that XCD's logical tiles
// x * per_xcd + slot, + workgroups per XCD, ... (tile order as tile_coords).
template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_persistent_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int total = tiles_m * tiles_n;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_wg = gridDim.x >> 3;
  const int share = (total + 7) >> 3;
  const int lo = xcd * share, hi = min(lo + share, total);
  const auto job_of = [&](int t) {
    int tm, tn;
    tile_order(t, tiles_m, tiles_n, 4, tm, tn);
    TileJob jb;
    jb.ar.lo = tm * C::BM;
    jb.ar.end = min(jb.ar.lo + C::BM, args.m);
    jb.ar.last = jb.ar.end - 1;
    jb.n0 = tn * C::BN;
    jb.b_q = args.b_q;
    jb.b_s = args.b_s;
    return jb;
  };
  persistent_loop<C>(args, lo + slot, per_wg, hi, job_of, (uint8_t MXFP4_LDS*)smem);
}

// Grouped persistent kernel.  The real tiles (counted from the sanitized
// offsets) are numbered expert by expert and, inside an expert, in the order
// of expert_tile: the m-tiles that share one weight panel are neighbours,
// dealt to neighbouring workgroups of one XCD in the same round, so the later
// readers of the panel can find it in that XCD's L2 (n-tile-major measured
// ~1 % faster than m-tile-major on a 64-expert MoE layer, the groups of four
// m-tiles another ~1.5 %).  The numbered tiles split evenly over the 8 XCDs
// as contiguous ranges, each range dealt round-robin to its XCD's workgroups.
template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_persistent_kernel(GemmArgs args, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int total = count_mtiles(args.offsets, args.groups, args.m, C::BM) * tiles_n;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_wg = gridDim.x >> 3;
  const int share = (total + 7) >> 3;
  const int lo = xcd * share, hi = min(lo + share, total);
  const int64_t kb = args.k / 2, ks = args.k / 32;
  const auto job_of = [&](int t) {
    TileJob jb;
    ExpertTiles e;
    int tn = 0;
    if (find_expert(args.offsets, args.groups, args.m, C::BM, t / tiles_n, e)) {
      const int local = t - e.first * tiles_n;   // in [0, cnt * tiles_n)
      int mi;
      expert_tile(local, e.cnt, tiles_n, tn, mi);
      jb.ar.lo = e.lo + mi * C::BM;
      jb.ar.end = min(e.hi, jb.ar.lo + C::BM);
      jb.ar.last = jb.ar.end - 1;
    } else {
      // unreachable for t < total (the counts agree); an empty row range stores nothing
      e.g = 0;
      jb.ar.lo = 0;
      jb.ar.end = 0;
      jb.ar.last = 0;
    }
    jb.n0 = tn * C::BN;
    jb.b_q = args.b_q + (int64_t)e.g * args.n * kb;
    jb.b_s = args.b_s + (int64_t)e.g * args.n * ks;
    return jb;
  };
  persistent_loop<C>(args, lo + slot, per_wg, hi, job_of, (uint8_t MXFP4_LDS*)smem);
}

using Cfg256 = TileCfg<256, 256, 2, 4>;
using Cfg128 = TileCfg<128, 128, 2, 2>;
using CfgW4A8 = TileCfg<128, 256, 2, 4, true>;
// Both operands MXFP8: 128-K stages keep a stage at 64 KiB for 256 x 256
// tiles.  An FP8 fragment is twice an FP4 one, so 8 waves of 128 x 64 would
// need more than their 256 registers; 4 waves (one per SIMD) of 128 x 128
// keep the 256 accumulators in the accumulator registers instead, and read
// a third fewer LDS bytes per MFMA.
using Cfg8x8_256 = TileCfg<256, 256, 2, 2, false, true>;
using Cfg8x8_128 = TileCfg<128, 128, 2, 2, false, true>;

// Dynamic LDS above 64 KiB has to be allowed per kernel.
template <class K>
hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// The copy path reads 16-byte scale pieces: k % 512 == 0 and 16-byte aligned
// scale arrays (row starts are then aligned too).  Interleaved scales exist
// only on the copy path (the register path reads row-major scales).
bool use_copy_path(const GemmArgs& args) {
  return args.k % 512 == 0 && ((reinterpret_cast<uintptr_t>(args.a_s) | reinterpret_cast<uintptr_t>(args.b_s)) & 15) == 0;
}

bool scale_layout_ok(const GemmArgs& args) { return !args.scale_il || use_copy_path(args); }

// GENERIC = false: the configuration has no register path (k % 512 != 0 or
// unaligned scale arrays are refused with hipErrorInvalidValue).
template <class C, bool GENERIC = true>
hipError_t launch_dense(const GemmArgs& args, hipStream_t stream) {
  const int tiles_m = (args.m + C::BM - 1) / C::BM;
  const int tiles_n = (args.n + C::BN - 1) / C::BN;
  const size_t lds = C::LDS_BYTES;
  const int64_t blocks = (int64_t)tiles_m * tiles_n;
  if (!grid_fits(blocks, C::THREADS)) return hipErrorInvalidConfiguration;
  if (!scale_layout_ok(args)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  if (use_copy_path(args)) {
    hipError_t e = allow_lds(gemm_tile_kernel<C, true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_tile_kernel<C, true>), grid, dim3(C::THREADS), lds, stream, args, tiles_m, tiles_n);
  } else if constexpr (GENERIC) {
    hipError_t e = allow_lds(gemm_tile_kernel<C, false>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_tile_kernel<C, false>), grid, dim3(C::THREADS), lds, stream, args, tiles_m, tiles_n);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class C>
hipError_t launch_grouped(const GemmArgs& args, hipStream_t stream) {
  const int64_t mt_bound = (args.m + C::BM - 1) / C::BM + args.groups;
  const int tiles_n = (args.n + C::BN - 1) / C::BN;
  const size_t lds = C::LDS_BYTES;
  const int64_t blocks = (mt_bound * tiles_n + 7) / 8 * 8;
  if (!grid_fits(blocks, C::THREADS)) return hipErrorInvalidConfiguration;
  if (!scale_layout_ok(args)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  if (use_copy_path(args)) {
    hipError_t e = allow_lds(grouped_tile_kernel<C, true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_tile_kernel<C, true>), grid, dim3(C::THREADS), lds, stream, args, tiles_n);
  } else {
    hipError_t e = allow_lds(grouped_tile_kernel<C, false>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_tile_kernel<C, false>), grid, dim3(C::THREADS), lds, stream, args, tiles_n);
  }
  return hipGetLastError();
}

// The persistent kernels need the copy path with an even number of scale
// groups per tile (k % 1024 == 0).
bool persistent_ok(const GemmArgs& args) { return use_copy_path(args) && args.k % 1024 == 0; }

// Workgroups of a persistent launch: one per compute unit, a multiple of 8
// (one per XCD slot), capped by `max_wgs` (0: no cap) and by 8 x the tiles one
// XCD takes.
int persistent_grid(int num_cus, int max_wgs, int64_t tiles) {
  int wgs = max(8, num_cus & ~7);
  if (max_wgs > 0) wgs = min(wgs, max(8, max_wgs & ~7));
  const int64_t per_xcd = (tiles + 7) / 8;
  if (8 * per_xcd < wgs) wgs = (int)(8 * per_xcd);
  return max(8, wgs);
}

template <class C>
hipError_t launch_dense_persistent(const GemmArgs& args, int num_cus, int max_wgs, hipStream_t stream) {
  if (!persistent_ok(args)) return hipErrorInvalidValue;
  const int tiles_m = (args.m + C::BM - 1) / C::BM;
  const int tiles_n = (args.n + C::BN - 1) / C::BN;
  const int grid = persistent_grid(num_cus, max_wgs, (int64_t)tiles_m * tiles_n);
  hipError_t e = allow_lds(gemm_persistent_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_persistent_kernel<C>), dim3(grid), dim3(C::THREADS), C::LDS_BYTES, stream, args, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

template <class C>
hipError_t launch_grouped_persistent(const GemmArgs& args, int num_cus, int max_wgs, hipStream_t stream) {
  if (!persistent_ok(args)) return hipErrorInvalidValue;
  const int64_t mt_bound = (args.m + C::BM - 1) / C::BM + args.groups;
  const int tiles_n = (args.n + C::BN - 1) / C::BN;
  const int grid = persistent_grid(num_cus, max_wgs, mt_bound * tiles_n);
  hipError_t e = allow_lds(grouped_persistent_kernel<C>, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((grouped_persistent_kernel<C>), dim3(grid), dim3(C::THREADS), C::LDS_BYTES, stream, args,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace

bool gemm_persistent_supported(const GemmArgs& args) { return persistent_ok(args); }

hipError_t launch_gemm_tile_persistent(const GemmArgs& args, int num_cus, int max_wgs, hipStream_t stream) {
  return launch_dense_persistent<Cfg256>(args, num_cus, max_wgs, stream);
}

hipError_t launch_grouped_gemm_tile_persistent(const GemmArgs& args, int num_cus, int max_wgs, hipStream_t stream) {
  return launch_grouped_persistent<Cfg256>(args, num_cus, max_wgs, stream);
}

hipError_t launch_grouped_gemm_w4a8_tile_persistent(const GemmArgs& args, int num_cus, int max_wgs,
                                                    hipStream_t stream) {
  return launch_grouped_persistent<CfgW4A8>(args, num_cus, max_wgs, stream);
}

hipError_t launch_gemm_tile(const GemmArgs& args, TileKind kind, hipStream_t stream) {
  return kind == kTile256 ? launch_dense<Cfg256>(args, stream) : launch_dense<Cfg128>(args, stream);
}

hipError_t launch_grouped_gemm_tile(const GemmArgs& args, TileKind kind, hipStream_t stream) {
  return kind == kTile256 ? launch_grouped<Cfg256>(args, stream) : launch_grouped<Cfg128>(args, stream);
}

hipError_t launch_gemm_w4a8_tile(const GemmArgs& args, hipStream_t stream) {
  return launch_dense<CfgW4A8>(args, stream);
}

hipError_t launch_grouped_gemm_w4a8_tile(const GemmArgs& args, hipStream_t stream) {
  return launch_grouped<CfgW4A8>(args, stream);
}

hipError_t launch_gemm_mxfp8_tile(const GemmArgs& args, TileKind kind, hipStream_t stream) {
  // the 256 x 256 configuration has no register path: other k take 128 x 128 tiles
  if (kind == kTile256 && use_copy_path(args)) return launch_dense<Cfg8x8_256, false>(args, stream);
  return launch_dense<Cfg8x8_128>(args, stream);
}

}  // namespace mxfp4
