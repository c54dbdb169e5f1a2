"""CPU oracle of the sigmoid-routed MoE FFN: test infrastructure only (see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (ALPHA_K2, E4M3_TABLE, FP8_BLOCK, KERNEL_BF16_POINTS, KERNEL_BF16_POINTS_TWO_PART,
                         PAGE_BF16_POINTS, dequant_fp8_blocks, e4m3_value,
                         gate_matrix, moe_block, moe_dense, moe_latent, moe_param_count,
                         moe_param_shapes, moe_sparse, permute, rmsnorm, round_bf16, route,
                         sigmoid, silu, swiglu)
