"""MI355X-native single-GPU MoE layer: route -> permute -> grouped SwiGLU FFN -> combine.

The compute runs in the HIP library `libmoe.so` (built from `csrc/`); the functions exported
here only marshal torch tensors into its C ABI. Loading is deferred to the first call so that
host-only helpers (`traffic`) import without a GPU; a missing library raises at that call.
"""
from .binding import (  # noqa: F401
    MoeError, Workspace, library_path, load_library, moe_combine, moe_grouped_ffn, moe_layer,
    moe_layer_workspace_size, moe_ffn_workspace_size, moe_permute, moe_permute_workspace_size,
    moe_route, moe_expert_capacity, moe_route_gemm, moe_route_gemm_workspace_size,
    moe_block_weights,
)
