"""MI355X (gfx950) W4A16 routed-expert MoE layer: HIP kernels behind a C ABI
(``include/moe_w4a16.h``), a ctypes binding with the same entry-point names,
and a thin layer driver.  PyTorch is used for device memory and streams only."""
from . import _lib
from ._lib import (MOE_ACT_NONE, MOE_ACT_SWIGLU, MOE_DECODE_WORKSPACE_BYTES, MOE_DOWN_COMBINE_MAX_TOKENS,
                   MOE_TILED_MIN_TOKENS, MoeError, MoeLayerDesc, moe_combine, moe_gen_fp16_scales,
                   moe_gen_int4_codes, moe_permute, moe_route, moe_route_permute, moe_row_sums,
                   moe_w4a16_decode_token, moe_w4a16_decode_token_supported, moe_w4a16_down_combine,
                   moe_w4a16_grouped_gemm, moe_w4a16_prepack, moe_mxfp4_grouped_gemm, moe_mxfp4_prepack,
                   moe_gen_ue8m0_scales, moe_mxfp4_decode_token, moe_w4a8_decode_token, moe_workspace_bytes,
                   moe_route_permute_noalloc, moe_act_quant_fp8, moe_act_quant_fp8_dequant, moe_w4a8_grouped_gemm,
                   moe_fp8_block_gemm, moe_fp8_prepack)
from .layer import Buffers, DecodeTimeout, ExpertWeights, MoELayer, generate_weights, prepack, upload_weights

__all__ = ["moe_act_quant_fp8", "moe_act_quant_fp8_dequant", "moe_w4a8_grouped_gemm", "moe_fp8_block_gemm", "moe_fp8_prepack",
           "moe_workspace_bytes", "moe_route_permute_noalloc", "MOE_ACT_NONE", "MOE_ACT_SWIGLU", "MOE_TILED_MIN_TOKENS", "MoeError", "MoeLayerDesc",
           "moe_route", "moe_permute", "moe_route_permute", "moe_w4a16_grouped_gemm", "moe_row_sums",
           "moe_w4a16_down_combine", "MOE_DOWN_COMBINE_MAX_TOKENS", "moe_w4a16_decode_token",
           "moe_w4a16_decode_token_supported", "MOE_DECODE_WORKSPACE_BYTES", "moe_combine", "moe_w4a16_prepack", "moe_gen_int4_codes",
           "moe_gen_fp16_scales", "moe_mxfp4_grouped_gemm", "moe_mxfp4_prepack", "moe_gen_ue8m0_scales", "moe_mxfp4_decode_token", "moe_w4a8_decode_token", "Buffers", "DecodeTimeout", "ExpertWeights", "MoELayer", "generate_weights",
           "prepack", "upload_weights"]
