"""CPU oracle (test infrastructure only; see mxfp4_oracle's docstring)."""
from .mxfp4_oracle import *  # noqa: F401,F403
from .mxfp4_oracle import (  # noqa: F401
    BLOCK, E2M1_TABLE, E2M1_MAGNITUDES, e2m1_value, e8m0_value,
    bf16_bits_to_f64, f64_to_bf16_bits, shared_exponent, encode_e2m1_magnitude,
    quantize_block_values, pack_codes, unpack_codes, quantize, dequantize,
    gemm_nt, gemm_nt_f32, grouped_gemm_nt, round_output_bf16, floored_max_rel,
)
from .mxfp8_oracle import (  # noqa: F401
    E4M3_TABLE, E4M3_MAGNITUDES, E4M3_MAX, e4m3_value, shared_exponent_e4m3, encode_e4m3_magnitude,
    quantize_block_values_e4m3, quantize_mxfp8, dequantize_mxfp8, gemm_w4a8_nt, gemm_mxfp8_nt,
)
from .moe_oracle import (  # noqa: F401
    route_topk, permute, quantize_scatter, quantize_scatter_mxfp8, combine, combine_abs,
)
from .producers_oracle import (  # noqa: F401
    add_residual, rmsnorm_f64, rmsnorm_bf16, swiglu_f64, swiglu_bf16,
)
from .nvfp4_oracle import (  # noqa: F401
    NVFP4_BLOCK, global_scales, quantize_nvfp4, dequantize_nvfp4, gemm_nvfp4_nt,
)
