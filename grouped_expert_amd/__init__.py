"""grouped_expert_amd: the single-GPU MoE routed-expert layer on MI355X.

The compute lives in ``libgrouped_expert_amd.so`` (hand-written HIP kernels
for gfx950 behind the C ABI of ``include/moe.h``); this package only
marshals torch tensors into those calls.  Importing it fails when the
library has not been built.
"""
from . import binding  # noqa: F401
from .binding import (MOE_BF16, MOE_F32, MOE_FP8_B128, MOE_FP8_ROW,  # noqa: F401
                      MOE_GATING_SIGMOID_BIAS_GROUP_TOP2, MOE_GATING_SOFTMAX_GROUP_LIMITED, MOE_GATING_SOFTMAX_TOPK,
                      MOE_GATING_SOFTMAX_TOPK_RENORM, MoEError, combine_backward, dequantize_fp8, expand_rows,
                      grouped_swiglu, grouped_swiglu_backward, header_rows, lib, new_act, new_flags, permute,
                      pool_height,
                      pool_pack, quantize_fp8, recv_compact, route_topk, route_topk_grouped, row_bytes, strerror,
                      unpermute_combine)
from .layer import loopback_wave, moe_layer, moe_layer_backward  # noqa: F401
