"""Latent-MoE layer forward for MI355X (gfx950): HIP kernels behind a C ABI.

The compute path lives in ``csrc/`` (built into ``liblatent_moe.so``); this
package only binds it (``binding``) and builds it (``build``).
"""
from .binding import (LMOE_BF16, LMOE_F32, LMOE_MXFP4, LatentMoE, LatentMoEError, latent_moe_create,
                      latent_moe_debug_views, latent_moe_destroy, latent_moe_forward,
                      latent_moe_last_error, latent_moe_set_profiling, latent_moe_stage_times,
                      latent_moe_workspace_bytes, make_config)

__all__ = [
    "LatentMoE", "LatentMoEError", "latent_moe_create", "latent_moe_forward", "latent_moe_destroy",
    "latent_moe_last_error", "latent_moe_workspace_bytes", "latent_moe_set_profiling",
    "latent_moe_stage_times", "latent_moe_debug_views", "make_config",
    "LMOE_F32", "LMOE_BF16", "LMOE_MXFP4",
]
