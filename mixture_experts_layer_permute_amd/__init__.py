"""MoE layer forward and backward on one MI355X (gfx950), behind the C ABI
of ``include/moe.h``.

Every function here has the name of a C entry point and only marshals
arguments: it takes torch tensors that live on the GPU, allocates outputs
and workspaces when the caller gives none, and passes raw device pointers
and the current HIP stream to ``libmoe.so``.  Every step of the layer runs
in the library's HIP kernels.  ``MoELayer`` preallocates all buffers of one
layer shape and chains the calls (forward, then backward).
"""
from ._lib import (MOE_ACT_GELU, MOE_ACT_SWIGLU, MOE_BF16, MOE_F32,  # noqa: F401
                   MoEError, load)
from .ops import (moe_combine, moe_combine_bwd, moe_expert_ffn_bwd,  # noqa: F401
                  moe_expert_ffn_fwd, moe_expert_ffn_fwd_gather,
                  moe_expert_ffn_fwd_noalloc,
                  moe_expert_ffn_bwd_gather, moe_gate_topk, moe_gate_topk_bwd,
                  moe_permute, moe_unpermute_grad, moe_init,
                  moe_set_overlap)
from .layer import ChunkedMoELayer, MoELayer, OffloadedMoELayer  # noqa: F401
