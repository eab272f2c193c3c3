"""grouped_expert_amd: the single-GPU MoE routed-expert layer on MI355X.

The compute lives in ``libgrouped_expert_amd.so`` (hand-written HIP kernels
for gfx950 behind the C ABI of ``include/moe.h``); this package only
marshals torch tensors into those calls.  Importing it fails when the
library has not been built.
"""
from .binding import (MOE_BF16, MOE_F32, MoEError, grouped_swiglu, lib, new_flags, permute, pool_pack,  # noqa: F401
                      recv_compact, route_topk, strerror, unpermute_combine)
from .layer import loopback_wave, moe_layer  # noqa: F401
