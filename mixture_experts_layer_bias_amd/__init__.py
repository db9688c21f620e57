"""MI355X (gfx950) MoE layer with zero-computation experts.

The layer runs in hand-written HIP kernels behind the C ABI of
include/moe_zc.h (libmoe_zc.so, built in-tree by ``_build.build()``); this
package is its thin Python binding.
"""
from .api import (  # noqa: F401
    AUX_KEYS, MoeZcError, PidState, StageEvents, alloc_aux, moe_zc_abi_version,
    moe_zc_bias_update, moe_zc_forward, moe_zc_forward_packed, moe_zc_pack_expert_weights,
    moe_zc_packed_expert_bytes, moe_zc_route, moe_zc_status_string, moe_zc_workspace_size,
    moe_zc_forward_packed_fp8, moe_zc_pack_expert_weights_fp8, moe_zc_packed_fp8_expert_bytes,
    moe_zc_quantize_mx, moe_zc_workspace_size_fp8, BWD_AUX_KEYS, moe_zc_backward,
    moe_zc_backward_workspace_size, moe_zc_transpose_expert_weights,
    moe_zc_transposed_expert_bytes, moe_zc_forward_packed_noalloc,
)
from ._lib import LIB_PATH, STAGE_NAMES  # noqa: F401
