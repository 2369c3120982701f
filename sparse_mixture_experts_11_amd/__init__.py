"""MI355X-native sparse mixture-of-experts feed-forward layer: the forward
pass, the Quantile Balancing bias update and the backward pass (router and
experts).

The compute path is libmoe.so (hand-written HIP for gfx950, C ABI in
include/moe.h); this package is its thin Python binding.
"""
from .api import (QB_EXACT, QB_HISTOGRAM, MoeError, backward_workspace,  # noqa: F401
                  make_desc, moe_backward_workspace_bytes, moe_experts_backward,
                  moe_capacity_from_factor, moe_combine, moe_desc_init, moe_dispatch,
                  moe_expert_ffn, moe_expert_ffn_scaled, moe_forward, moe_forward_noalloc,
                  moe_forward_traced,
                  moe_latent_backward,
                  moe_qb_update, moe_route, moe_route_backward, moe_route_biased,
                  moe_stage_names, moe_status_string, moe_workspace_bytes, workspace)
from ._lib import LibraryMissing, SO_PATH, load  # noqa: F401
