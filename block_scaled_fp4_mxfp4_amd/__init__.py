"""MI355X (gfx950) MXFP4 engine: BF16 -> MXFP4 quantization, block-scaled FP4 NT GEMM,
grouped per-expert GEMM (also on an interleaved scale layout), a decode GEMM on prepacked weights, BF16 -> MXFP8 quantization, W4A8 GEMMs
(MXFP8 A x MXFP4 B) and the MXFP8 x MXFP8 GEMM, and the MoE steps around the grouped GEMM (top-k routing,
expert-sorted permutation, scatter-quantize, combine) and fused producers that
emit MXFP4 (residual add + RMSNorm, SwiGLU), and NVFP4 (two-level: UE4M3 per
16 elements, fp32 per row) quantization and GEMM, as hand-written HIP kernels
behind a C ABI (include/mxfp4.h, include/mxfp8.h, include/mxfp4_moe.h,
include/mxfp4_producers.h, include/nvfp4.h).  The Python layer is a thin ctypes binding."""
from .binding import (  # noqa: F401
    MXFP4Error, load_library, mxfp4_quantize, mxfp8_quantize, mxfp4_gemm_nt, mxfp4_grouped_gemm_nt, workspace,
    mxfp8_gemm_w4a8_nt, mxfp8_grouped_gemm_w4a8_nt, mxfp8_gemm_nt, mxfp8_gemm_w4a8_nt_prepacked,
    mxfp4_moe_route, mxfp4_moe_permute, mxfp4_moe_quantize_scatter, mxfp8_moe_quantize_scatter, mxfp4_moe_combine,
    mxfp4_rmsnorm_quantize, mxfp4_swiglu_quantize, nvfp4_quantize, nvfp4_gemm_nt,
    mxfp4_prepacked_weight_size, mxfp4_prepack_weight, mxfp4_gemm_nt_prepacked, mxfp4_gemm_nt_prepacked_ab,
    mxfp4_quantize_prepacked, mxfp4_scales_interleave, mxfp4_quantize_interleaved, mxfp4_gemm_nt_interleaved,
    mxfp4_grouped_gemm_nt_interleaved, mxfp4_moe_quantize_scatter_interleaved, mxfp8_quantize_prepacked,
    mxfp8_gemm_w4a8_nt_prepacked_ab, mxfp8_quantize_interleaved, mxfp8_gemm_w4a8_nt_interleaved,
    mxfp8_grouped_gemm_w4a8_nt_interleaved, mxfp8_gemm_nt_interleaved, mxfp8_moe_quantize_scatter_interleaved,
    LIB_PATH, EXPORTED, KERNELS,
)
