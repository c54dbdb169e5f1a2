"""MI355X-native sigmoid-routed MoE FFN layer (Kimi K2 / DeepSeek-V3 style).

The computation lives in libmoe.so (HIP kernels for gfx950, C ABI in include/moe.h);
this package is its ctypes binding.
"""
from .binding import (EXPORTS, LIB_PATH, MOE_EHIP, MOE_EINVAL, MOE_ESCRATCH, MOE_EUNSUPPORTED,
                      MOE_EWORKSPACE, MOE_OK, NOALLOC_SCRATCH_BYTES, HSPLIT_MAX_D_EXPERT, HSPLIT_MAX_TOP_K, MoeDims, h_width, MoeError, MoeFp8Weights, block_workspace, dims_for,
                      fp8_weights, latent_workspace, lib, moe_expert_down_fp8,
                      moe_expert_gate_up_fp8, moe_forward_fp8,
                      moe_block_workspace_bytes, moe_combine, moe_dims, moe_expert_down,
                      moe_expert_ffn, moe_expert_gate_up, moe_forward, moe_forward_block,
                      moe_forward_latent, moe_forward_noalloc, moe_latent_workspace_bytes, moe_permute, moe_route,
                      moe_workspace_bytes, moe_workspace_release, routing_in_workspace, status_str,
                      workspace)

__all__ = ["EXPORTS", "LIB_PATH", "MOE_EHIP", "MOE_EINVAL", "MOE_ESCRATCH", "MOE_EUNSUPPORTED",
           "MOE_EWORKSPACE", "MOE_OK", "NOALLOC_SCRATCH_BYTES", "HSPLIT_MAX_D_EXPERT", "HSPLIT_MAX_TOP_K", "h_width", "moe_forward_noalloc", "MoeDims", "MoeError", "MoeFp8Weights", "block_workspace", "dims_for",
           "fp8_weights", "latent_workspace", "moe_expert_down_fp8", "moe_expert_gate_up_fp8",
           "moe_forward_fp8",
           "lib", "moe_block_workspace_bytes", "moe_combine", "moe_forward_block",
           "moe_dims", "moe_expert_down", "moe_expert_ffn", "moe_expert_gate_up", "moe_forward",
           "moe_forward_latent", "moe_latent_workspace_bytes", "moe_permute", "moe_route",
           "moe_workspace_bytes", "moe_workspace_release", "routing_in_workspace", "status_str",
           "workspace"]
