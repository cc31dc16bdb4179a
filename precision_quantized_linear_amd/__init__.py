"""MI355X (gfx950) quantized linear: fp8r and nvfp4 (BFL schemes) with an optional
SVDQuant low-rank branch and smoothing, its INT4 variant, and the weight-only
4-bit (awq_w4a16) linear, with GELU and fused-QKV epilogues and the fused GELU MLP.
The HIP library libqpl.so does the work; this package is its thin Python binding."""
from ._binding import (EXPORTS, KERNELS, LIB_PATH, QPL_ACT_GELU_TANH, QPL_ACT_NONE, QPL_FP8R,  # noqa: F401
                       QPL_INT4, QPL_NVFP4, Epilogue, Nvfp4Layer, QPLError, amax_bf16, dequant_weight, load,
                       nvfp4_global_scale, qlinear_awq_w4a16, qlinear_fp8r, qlinear_fp8r_noalloc, qlinear_int4, qlinear_mlp_nvfp4,
                       qlinear_mlp_nvfp4_workspace_bytes, qlinear_nvfp4, qlinear_workspace_bytes, quant_act_fp8_row,
                       quant_act_int4, quant_act_nvfp4, quant_weight_awq, timing_collect, timing_enable,
                       timing_select)
