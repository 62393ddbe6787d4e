"""MI355X-native grouped expert MLP (permute -> grouped GEMM -> ScaledSwiGLU*prob
-> grouped GEMM -> combine) in BF16 and MXFP8 (forward and backward) and in
per-tensor-scaled FP8 (forward), behind the C ABI of libmoe.so.

The functions below are thin ctypes wrappers; all computation happens in the
library's HIP kernels for gfx950.
"""
from ._lib import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_MXFP8_E4M3, EXPORTS, MoeError, load, fp8_tensor_quantize,
                   moe_grouped_mlp_bwd, moe_grouped_mlp_fwd, moe_grouped_mlp_fwd_loop, moe_permute,
                   moe_permute_noalloc, moe_read_device_error, moe_route_permute, moe_route_topk, mxfp8_quantize,
                   mxfp8_quantize_weights, quantize_weights, set_tile_stats, tile_stats_new, tile_stats_summary, mfma_probe,
                   load_probe,
                   LIB_PATH)

__all__ = [
    "MOE_BF16", "MOE_F32", "MOE_FP8_E4M3", "MOE_MXFP8_E4M3", "EXPORTS", "MoeError", "load",
    "fp8_tensor_quantize", "moe_grouped_mlp_bwd", "moe_grouped_mlp_fwd", "moe_grouped_mlp_fwd_loop", "moe_permute",
    "moe_permute_noalloc", "moe_read_device_error", "moe_route_permute", "moe_route_topk", "mxfp8_quantize",
    "mxfp8_quantize_weights", "quantize_weights", "set_tile_stats", "tile_stats_new", "tile_stats_summary", "mfma_probe", "load_probe",
    "LIB_PATH",
]
